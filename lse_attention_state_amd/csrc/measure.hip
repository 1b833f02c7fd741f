// A plain streaming read of one buffer for gfx950: the practical HBM read
// rate of this device, measured beside the kernels so that their fractions of
// the 8 TB/s peak can be read against what a kernel that only reads reaches.
//
// Each workgroup reads one contiguous block of kUnroll * 256 16-byte chunks
// with the non-temporal hint (as the merge kernels do), all of a lane's loads
// in flight at once; there is no grid-stride loop. (On MI355X, contiguous
// per-workgroup blocks read 1 GiB at about 6.9 TB/s; a grid-stride loop whose
// steps jump by the grid's size reached 5.6-6.2 TB/s.) The chunks' 32-bit
// words are XOR-ed together, so that the result depends on every byte and can
// be checked exactly; each workgroup folds its lanes and XORs its value into
// *xor_out with one vector atomic.
#include "common.h"
#include "launch.h"

namespace mi {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // chunks per lane: one 32 KiB block per workgroup

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4_t* __restrict__ x,
                                                               int64_t n16,
                                                               uint32_t* __restrict__ xor_out) {
  __shared__ uint32_t part[kThreads / 64];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kThreads * kUnroll) + threadIdx.x;
  u32x4_t c[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * kThreads;
    c[u] = i < n16 ? __builtin_nontemporal_load(x + i) : u32x4_t{0, 0, 0, 0};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) acc ^= c[u].x ^ c[u].y ^ c[u].z ^ c[u].w;
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1)
    acc ^= __builtin_bit_cast(uint32_t, shfl_xor(__builtin_bit_cast(float, acc), sh));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) a ^= part[w];
    if (a != 0) atomicXor(xor_out, a);
  }
}

}  // namespace

hipError_t launch_stream_read(const void* x, int64_t bytes, uint32_t* xor_out, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  const int64_t blocks = (n16 + kThreads * kUnroll - 1) / (kThreads * kUnroll);
  if (!grid_fits(blocks, kThreads)) return hipErrorInvalidConfiguration;
  stream_read_kernel<<<dim3(static_cast<unsigned>(blocks)), kThreads, 0, st>>>(
      static_cast<const u32x4_t*>(x), n16, xor_out);
  return hipGetLastError();
}

}  // namespace mi
