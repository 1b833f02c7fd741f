// Plain, slow CPU oracle for attention-state merging and split-KV paged decode.
//
// TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's
// cpu_baseline leg load this library. The product path (libmi.so and its Python
// binding) never links, imports or calls it, and it shares no code, header,
// table or helper with the HIP path. Every floating-point step is done in
// double precision with the host libm; fp16 and bf16 inputs are decoded by this
// file's own codecs.
//
// What is computed, and where it is defined (page titles and sections):
//  * "F2 hints: merge_state, base-2 LSE merge", section 1 (the state (v, s)) and
//    section 2 (base-2 LSE): a state is the softmax-normalised output over a key
//    subset plus that subset's log2-sum-exp.
//  * same page, sections 3 and 4: merging two states and N states; layouts
//    v[S,H,D] / s[S,H] and v[S,N,H,D] / s[S,N,H].
//  * same page, section 5: an empty key set is (v = 0, s = -inf).
//  * "FlashAttention's empty-row LSE", section 2.2: an incoming NaN or +inf
//    LSE is treated as -inf (no weight).
//  * same page, section 0 (the definitions of Z, L, P, O): plain softmax
//    attention; used here for unsplit decode and for each split's partial.
//  * "L3 hints: split-KV decode and LSE merge", section 2: page ranges of a
//    split; section 4: an empty split writes (o = 0, lse = -inf); section 6: the
//    rule of thumb for the number of splits, and plan() giving sequences of
//    different lengths different numbers of splits.
//  * "FlashAttention's empty-row LSE", section 0 (table) and section 2.1: an
//    attention sink rescales the output by e^L / (e^L + e^sink) and adds the
//    sink to the LSE, i.e. it is a key of logit `sink` and value 0.
//  * "F2 hints", section 7: merge_state_in_place (here with a per-position
//    mask) and merge_states over many or variable-length index sets.
//
// Merges are written as the plain definition over the set E of non-empty states
// (an explicit branch, not a max trick): if E is empty the result is (0, -inf);
// otherwise m = max over E, w_i = 2^(s_i - m), v = sum w_i v_i / sum w_i,
// s = m + log2(sum w_i).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

enum { OR_F16 = 0, OR_BF16 = 1, OR_F32 = 2 };

const double kNegInf = -std::numeric_limits<double>::infinity();

// IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
double f16_bits_to_double(uint16_t h) {
  const int sign = h >> 15;
  const int e = (h >> 10) & 0x1f;
  const int f = h & 0x3ff;
  double mag;
  if (e == 0) {
    mag = std::ldexp(static_cast<double>(f), -24);          // subnormal: f * 2^-24
  } else if (e == 31) {
    mag = f ? std::numeric_limits<double>::quiet_NaN()
            : std::numeric_limits<double>::infinity();
  } else {
    mag = std::ldexp(static_cast<double>(1024 + f), e - 25);  // (1 + f/2^10) * 2^(e-15)
  }
  return sign ? -mag : mag;
}

// bfloat16 is the upper half of an IEEE binary32 pattern.
double bf16_bits_to_double(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

double load_elem(const void* base, int dtype, int64_t i) {
  switch (dtype) {
    case OR_F16: return f16_bits_to_double(static_cast<const uint16_t*>(base)[i]);
    case OR_BF16: return bf16_bits_to_double(static_cast<const uint16_t*>(base)[i]);
    default: return static_cast<double>(static_cast<const float*>(base)[i]);
  }
}

bool dtype_ok(int dtype) { return dtype == OR_F16 || dtype == OR_BF16 || dtype == OR_F32; }

// "FlashAttention's empty-row LSE", section 2.2: NaN and +inf mean "no weight".
double sanitize(double s) {
  if (std::isnan(s) || s == std::numeric_limits<double>::infinity()) return kNegInf;
  return s;
}

// Merge n states given as (s[i], v[i*D .. i*D+D)) by the plain definition over
// the non-empty set E. s values must already be sanitised.
void merge_definition(int n, const double* s, const double* v, int D, double* v_out,
                      double* s_out) {
  bool any = false;
  double m = kNegInf;
  for (int i = 0; i < n; ++i) {
    if (s[i] == kNegInf) continue;  // not in E: contributes nothing, even if v is NaN
    if (!any || s[i] > m) m = s[i];
    any = true;
  }
  if (!any) {
    for (int d = 0; d < D; ++d) v_out[d] = 0.0;
    *s_out = kNegInf;
    return;
  }
  double z = 0.0;
  std::vector<double> acc(D, 0.0);
  for (int i = 0; i < n; ++i) {
    if (s[i] == kNegInf) continue;
    const double w = std::exp2(s[i] - m);
    z += w;
    for (int d = 0; d < D; ++d) acc[d] += w * v[static_cast<int64_t>(i) * D + d];
  }
  for (int d = 0; d < D; ++d) v_out[d] = acc[d] / z;
  *s_out = m + std::log2(z);
}

template <typename F>
void parallel_rows(int64_t rows, int threads, F fn) {
  if (threads <= 0) threads = static_cast<int>(std::max(1u, std::thread::hardware_concurrency()));
  if (rows < threads) threads = static_cast<int>(std::max<int64_t>(rows, 1));
  if (threads == 1) {
    for (int64_t r = 0; r < rows; ++r) fn(r);
    return;
  }
  std::vector<std::thread> pool;
  pool.reserve(threads);
  for (int t = 0; t < threads; ++t) {
    pool.emplace_back([=, &fn]() {
      for (int64_t r = t; r < rows; r += threads) fn(r);
    });
  }
  for (auto& th : pool) th.join();
}

// "L3 hints", section 2: pages of a split, [p0, p1); empty when p1 <= p0.
void split_pages(int ctx, int page, int splits, int k, int* p0, int* p1) {
  const int num_pages = ctx / page + (ctx % page != 0 ? 1 : 0);
  const int per_split = num_pages / splits + (num_pages % splits != 0 ? 1 : 0);
  const int start = k * per_split;
  int end = start + per_split;
  if (end > num_pages) end = num_pages;
  *p0 = start;
  *p1 = end;
}

struct DecodeArgs {
  const void* q;
  int q_dtype;
  const void* k_cache;
  const void* v_cache;
  int kv_dtype;
  const int32_t* page_table;
  int pt_stride;
  const int32_t* ctx_lens;
  int B, Hq, Hkv, D, page;
  double sm_scale;
};

// Plain softmax attention of query (b, hq) over tokens [t0, t1) of sequence b
// ("FlashAttention's empty-row LSE", section 0): x_t = scale * q.k_t,
// M = max x, Z = sum e^(x_t - M), o = sum e^(x_t - M) v_t / Z, L = M + ln Z.
// The state's s is L in base 2 (= L / ln 2). No tokens: (0, -inf).
void attend(const DecodeArgs& a, int b, int hq, int t0, int t1, double* o, double* s) {
  const int D = a.D;
  if (t1 <= t0) {
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    *s = kNegInf;
    return;
  }
  const int group = a.Hq / a.Hkv;
  const int hkv = hq / group;
  std::vector<double> q(D);
  for (int d = 0; d < D; ++d)
    q[d] = load_elem(a.q, a.q_dtype, (static_cast<int64_t>(b) * a.Hq + hq) * D + d);
  const int n = t1 - t0;
  std::vector<double> x(n);
  std::vector<int64_t> row(n);
  for (int i = 0; i < n; ++i) {
    const int t = t0 + i;
    const int64_t phys = a.page_table[static_cast<int64_t>(b) * a.pt_stride + t / a.page];
    row[i] = ((phys * a.Hkv + hkv) * a.page + t % a.page) * D;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += q[d] * load_elem(a.k_cache, a.kv_dtype, row[i] + d);
    x[i] = a.sm_scale * dot;
  }
  double M = x[0];
  for (int i = 1; i < n; ++i) M = std::max(M, x[i]);
  double Z = 0.0;
  std::vector<double> acc(D, 0.0);
  for (int i = 0; i < n; ++i) {
    const double e = std::exp(x[i] - M);
    Z += e;
    for (int d = 0; d < D; ++d) acc[d] += e * load_elem(a.v_cache, a.kv_dtype, row[i] + d);
  }
  for (int d = 0; d < D; ++d) o[d] = acc[d] / Z;
  *s = (M + std::log(Z)) / std::log(2.0);
}

bool decode_args_ok(const DecodeArgs& a) {
  return a.q && a.k_cache && a.v_cache && a.page_table && a.ctx_lens && a.B >= 0 && a.Hq > 0 &&
         a.Hkv > 0 && a.Hq % a.Hkv == 0 && a.D > 0 && a.page > 0 && dtype_ok(a.q_dtype) &&
         dtype_ok(a.kv_dtype);
}

}  // namespace

extern "C" {

// Codecs, exposed so the tests can check them against independent decoders.
int or_decode_f16(const uint16_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f16_bits_to_double(in[i]);
  return 0;
}

int or_decode_bf16(const uint16_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_bits_to_double(in[i]);
  return 0;
}

// Two states ("F2 hints", section 3): v_a, v_b [rows, D] of v_dtype; s_a, s_b [rows] fp32.
int or_merge_state(const void* va, const float* sa, const void* vb, const float* sb, int v_dtype,
                   int64_t rows, int D, double* v_out, double* s_out, int threads) {
  if (!va || !sa || !vb || !sb || !v_out || !s_out || rows < 0 || D <= 0 || !dtype_ok(v_dtype))
    return 1;
  parallel_rows(rows, threads, [&](int64_t r) {
    double s[2] = {sanitize(sa[r]), sanitize(sb[r])};
    std::vector<double> v(2 * static_cast<size_t>(D));
    for (int d = 0; d < D; ++d) {
      v[d] = load_elem(va, v_dtype, r * D + d);
      v[D + d] = load_elem(vb, v_dtype, r * D + d);
    }
    merge_definition(2, s, v.data(), D, v_out + r * D, s_out + r);
  });
  return 0;
}

// N states ("F2 hints", section 4): v [S,N,H,D], s [S,N,H] -> v_out [S,H,D], s_out [S,H].
// s[pos, n, h] sits at offset (pos*N + n)*H + h.
int or_merge_states(const void* v, const float* s, int v_dtype, int64_t S, int N, int H, int D,
                    double* v_out, double* s_out, int threads) {
  if (!v || !s || !v_out || !s_out || S < 0 || N <= 0 || H <= 0 || D <= 0 || !dtype_ok(v_dtype))
    return 1;
  parallel_rows(S * H, threads, [&](int64_t row) {
    const int64_t pos = row / H;
    const int h = static_cast<int>(row % H);
    std::vector<double> sv(N);
    std::vector<double> vv(static_cast<size_t>(N) * D);
    for (int n = 0; n < N; ++n) {
      const int64_t idx = (pos * N + n) * H + h;
      sv[n] = sanitize(s[idx]);
      for (int d = 0; d < D; ++d) vv[static_cast<size_t>(n) * D + d] = load_elem(v, v_dtype, idx * D + d);
    }
    merge_definition(N, sv.data(), vv.data(), D, v_out + row * D, s_out + row);
  });
  return 0;
}

int or_split_range(int ctx, int page, int splits, int k, int* p0, int* p1) {
  if (ctx < 0 || page <= 0 || splits <= 0 || k < 0 || k >= splits || !p0 || !p1) return 1;
  split_pages(ctx, page, splits, k, p0, p1);
  return 0;
}

// "L3 hints", section 6: make B*Hkv*splits a few times the number of compute
// units, with at least several pages per split; no split when B*Hkv is already
// large. Reading: the smallest of {1,4,16,64} reaching twice the CU count (else
// 64), then step down while a split would hold fewer than 8 pages.
int or_plan_splits(int B, int Hkv, const int32_t* ctx_lens, int page, int num_cus) {
  if (B <= 0 || Hkv <= 0 || !ctx_lens || page <= 0 || num_cus <= 0) return -1;
  const int options[4] = {1, 4, 16, 64};
  int max_pages = 0;
  for (int b = 0; b < B; ++b) {
    if (ctx_lens[b] < 0) return -1;
    const int np = ctx_lens[b] / page + (ctx_lens[b] % page != 0 ? 1 : 0);
    max_pages = std::max(max_pages, np);
  }
  int idx = 3;
  for (int i = 0; i < 4; ++i) {
    if (static_cast<int64_t>(B) * Hkv * options[i] >= 2LL * num_cus) {
      idx = i;
      break;
    }
  }
  while (idx > 0) {
    const int sp = options[idx];
    const int per_split = max_pages / sp + (max_pages % sp != 0 ? 1 : 0);
    if (per_split >= 8) break;
    --idx;
  }
  return options[idx];
}

// Unsplit decode: for each (b, hq), attention over tokens [0, ctx_lens[b]).
// o [B,Hq,D], s [B,Hq] (base-2 LSE).
int or_attention(const void* q, int q_dtype, const void* k_cache, const void* v_cache,
                 int kv_dtype, const int32_t* page_table, int pt_stride, const int32_t* ctx_lens,
                 int B, int Hq, int Hkv, int D, int page, double sm_scale, double* o, double* s,
                 int threads) {
  DecodeArgs a{q, q_dtype, k_cache, v_cache, kv_dtype, page_table, pt_stride, ctx_lens,
               B, Hq, Hkv, D, page, sm_scale};
  if (!decode_args_ok(a) || !o || !s) return 1;
  parallel_rows(static_cast<int64_t>(B) * Hq, threads, [&](int64_t row) {
    const int b = static_cast<int>(row / Hq);
    const int hq = static_cast<int>(row % Hq);
    attend(a, b, hq, 0, ctx_lens[b], o + row * D, s + row);
  });
  return 0;
}

// Per-split partials ("L3 hints", sections 2-5): o_part [B,Hq,splits,D],
// lse_part [B,Hq,splits] (base 2). Split k covers pages [p0, p1), i.e. tokens
// [p0*page, min(p1*page, ctx)); an empty split is (0, -inf).
int or_split_partials(const void* q, int q_dtype, const void* k_cache, const void* v_cache,
                      int kv_dtype, const int32_t* page_table, int pt_stride,
                      const int32_t* ctx_lens, int B, int Hq, int Hkv, int D, int page,
                      double sm_scale, int splits, double* o_part, double* lse_part,
                      int threads) {
  DecodeArgs a{q, q_dtype, k_cache, v_cache, kv_dtype, page_table, pt_stride, ctx_lens,
               B, Hq, Hkv, D, page, sm_scale};
  if (!decode_args_ok(a) || splits <= 0 || !o_part || !lse_part) return 1;
  parallel_rows(static_cast<int64_t>(B) * Hq * splits, threads, [&](int64_t row) {
    const int k = static_cast<int>(row % splits);
    const int64_t bh = row / splits;
    const int b = static_cast<int>(bh / Hq);
    const int hq = static_cast<int>(bh % Hq);
    const int ctx = ctx_lens[b];
    int p0, p1;
    split_pages(ctx, page, splits, k, &p0, &p1);
    int t0 = p0 * page;
    int t1 = std::min(p1 * page, ctx);
    if (p1 <= p0) t1 = t0;
    attend(a, b, hq, t0, t1, o_part + row * D, lse_part + row);
  });
  return 0;
}

// Attention sink ("FlashAttention's empty-row LSE", section 0 and section 2.1):
// the sink of head h is a key with logit sink[h] (natural units) and value 0,
// i.e. the state (v = 0, s = sink[h] / ln 2); the result is the merge of the
// row's state with it. The sink is sanitised like any LSE (NaN, +inf -> no
// sink). v [rows, D] with rows = S*H, head h = row % H; s [rows].
int or_merge_sink(const void* v, const float* s, int v_dtype, int64_t rows, int H, int D,
                  const float* sink, double* v_out, double* s_out, int threads) {
  if (!v || !s || !sink || !v_out || !s_out || rows < 0 || H <= 0 || D <= 0 || !dtype_ok(v_dtype))
    return 1;
  parallel_rows(rows, threads, [&](int64_t r) {
    const double sk = static_cast<double>(sink[r % H]) / std::log(2.0);
    double sv[2] = {sanitize(s[r]), sanitize(sk)};
    std::vector<double> vv(2 * static_cast<size_t>(D), 0.0);
    for (int d = 0; d < D; ++d) vv[d] = load_elem(v, v_dtype, r * D + d);
    merge_definition(2, sv, vv.data(), D, v_out + r * D, s_out + r);
  });
  return 0;
}

// Two states with a per-position mask (merge_state_in_place's optional mask,
// "F2 hints", section 7; its meaning is a reading, see the design notes):
// positions whose mask byte is 0 keep state a unchanged (not even sanitised);
// the others get merge(a, b). v [S,H,D], s [S,H], mask [S] (NULL: all merge).
int or_merge_state_masked(const void* va, const float* sa, const void* vb, const float* sb,
                          int v_dtype, int64_t S, int H, int D, const uint8_t* mask,
                          double* v_out, double* s_out, int threads) {
  if (!va || !sa || !vb || !sb || !v_out || !s_out || S < 0 || H <= 0 || D <= 0 ||
      !dtype_ok(v_dtype))
    return 1;
  parallel_rows(S * H, threads, [&](int64_t r) {
    if (mask != nullptr && mask[r / H] == 0) {
      for (int d = 0; d < D; ++d) v_out[r * D + d] = load_elem(va, v_dtype, r * D + d);
      s_out[r] = static_cast<double>(sa[r]);
      return;
    }
    double sv[2] = {sanitize(sa[r]), sanitize(sb[r])};
    std::vector<double> vv(2 * static_cast<size_t>(D));
    for (int d = 0; d < D; ++d) {
      vv[d] = load_elem(va, v_dtype, r * D + d);
      vv[D + d] = load_elem(vb, v_dtype, r * D + d);
    }
    merge_definition(2, sv, vv.data(), D, v_out + r * D, s_out + r);
  });
  return 0;
}

// Variable-length merge ("F2 hints", section 4 formula over index sets of any
// size): states v [total, H, D], s [total, H]; segment i (i < S) is the states
// indptr[i] .. indptr[i+1]-1 and merges into v_out [S, H, D], s_out [S, H]. An
// empty segment is the empty state.
int or_merge_states_varlen(const void* v, const float* s, int v_dtype, const int32_t* indptr,
                           int64_t S, int H, int D, double* v_out, double* s_out, int threads) {
  if (!v || !s || !indptr || !v_out || !s_out || S < 0 || H <= 0 || D <= 0 || !dtype_ok(v_dtype))
    return 1;
  for (int64_t i = 0; i < S; ++i)
    if (indptr[i] < 0 || indptr[i + 1] < indptr[i]) return 1;
  parallel_rows(S * H, threads, [&](int64_t row) {
    const int64_t seg = row / H;
    const int h = static_cast<int>(row % H);
    const int n = indptr[seg + 1] - indptr[seg];
    std::vector<double> sv(n > 0 ? n : 1);
    std::vector<double> vv(static_cast<size_t>(n > 0 ? n : 1) * D);
    for (int k = 0; k < n; ++k) {
      const int64_t idx = static_cast<int64_t>(indptr[seg] + k) * H + h;
      sv[k] = sanitize(s[idx]);
      for (int d = 0; d < D; ++d) vv[static_cast<size_t>(k) * D + d] = load_elem(v, v_dtype, idx * D + d);
    }
    merge_definition(n, sv.data(), vv.data(), D, v_out + row * D, s_out + row);
  });
  return 0;
}

// Per-sequence split counts ("L3 hints", section 6: plan() may give sequences
// of different lengths different numbers of splits). Reading: the uniform rule
// carried over to one page budget c shared by all sequences. The work items
// Hkv * sum_b max(1, ceil(np_b / c)) should reach twice the CU count with as
// few items as possible, so c is the largest value (up to the longest
// sequence's page count) whose items still reach it; a split keeps at least 8
// pages, so c never goes below 8. Sequence b gets max(1, ceil(np_b / c))
// splits. Returns c, or -1 on bad arguments; the counts go to counts[B].
// Found by counting down from the longest page count.
int or_plan_splits_varlen(int B, int Hkv, const int32_t* ctx_lens, int page, int num_cus,
                          int32_t* counts) {
  if (B <= 0 || Hkv <= 0 || !ctx_lens || page <= 0 || num_cus <= 0 || !counts) return -1;
  std::vector<int64_t> np(B);
  int64_t max_np = 0;
  for (int b = 0; b < B; ++b) {
    if (ctx_lens[b] < 0) return -1;
    np[b] = ctx_lens[b] / page + (ctx_lens[b] % page != 0 ? 1 : 0);
    max_np = std::max(max_np, np[b]);
  }
  auto items = [&](int64_t c) {
    int64_t w = 0;
    for (int b = 0; b < B; ++b) w += std::max<int64_t>(1, np[b] / c + (np[b] % c != 0 ? 1 : 0));
    return w * Hkv;
  };
  int64_t c = max_np;
  while (c > 8 && items(c) < 2LL * num_cus) --c;
  if (c < 8) c = 8;
  for (int b = 0; b < B; ++b)
    counts[b] = static_cast<int32_t>(std::max<int64_t>(1, np[b] / c + (np[b] % c != 0 ? 1 : 0)));
  return static_cast<int>(c);
}

// Partials with per-sequence splits: sequence b has n_b = indptr[b+1] -
// indptr[b] splits, and its split k (global index indptr[b] + k) takes the
// page range of the section-2 formula with n_b splits. o_part [total, Hq, D],
// lse_part [total, Hq] (base 2); a split without tokens is (0, -inf).
int or_split_partials_varlen(const void* q, int q_dtype, const void* k_cache, const void* v_cache,
                             int kv_dtype, const int32_t* page_table, int pt_stride,
                             const int32_t* ctx_lens, int B, int Hq, int Hkv, int D, int page,
                             double sm_scale, const int32_t* indptr, double* o_part,
                             double* lse_part, int threads) {
  DecodeArgs a{q, q_dtype, k_cache, v_cache, kv_dtype, page_table, pt_stride, ctx_lens,
               B, Hq, Hkv, D, page, sm_scale};
  if (!decode_args_ok(a) || !indptr || !o_part || !lse_part || indptr[0] != 0) return 1;
  for (int b = 0; b < B; ++b)
    if (indptr[b + 1] <= indptr[b]) return 1;
  const int total = indptr[B];
  std::vector<int> owner(total);
  for (int b = 0; b < B; ++b)
    for (int i = indptr[b]; i < indptr[b + 1]; ++i) owner[i] = b;
  parallel_rows(static_cast<int64_t>(total) * Hq, threads, [&](int64_t row) {
    const int i = static_cast<int>(row / Hq);
    const int hq = static_cast<int>(row % Hq);
    const int b = owner[i];
    int p0, p1;
    split_pages(ctx_lens[b], page, indptr[b + 1] - indptr[b], i - indptr[b], &p0, &p1);
    const int t0 = p0 * page;
    const int t1 = std::min(p1 * page, ctx_lens[b]);
    attend(a, b, hq, t0, t1 > t0 ? t1 : t0, o_part + row * D, lse_part + row);
  });
  return 0;
}

}  // extern "C"
