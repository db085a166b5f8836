// sv_probe.hip -- the plain streaming-read probe (a measurement aid, not part of the
// method): every 32 KiB chunk of a buffer read once by one 256-thread workgroup with
// 128-bit non-temporal loads, all issued before any is used, as the verification
// kernels' first pass reads logits.  Each workgroup's wrapping word sum goes to out[i].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_probe.h"

namespace {

constexpr int PNT = 256, PVPT = 8, PCHUNK = PNT * PVPT * 16;  // bytes per workgroup
typedef unsigned u32x4p __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(PNT) void k_read_probe(const u32x4p *buf, uint32_t *out) {
  __shared__ unsigned s_sum[PNT / 64];
  const int tid = threadIdx.x;
  const u32x4p *p = buf + (size_t)blockIdx.x * (PNT * PVPT) + tid;
  u32x4p w[PVPT];
#pragma unroll
  for (int k = 0; k < PVPT; ++k) w[k] = __builtin_nontemporal_load(p + k * PNT);
  unsigned s = 0;
#pragma unroll
  for (int k = 0; k < PVPT; ++k) s += w[k].x + w[k].y + w[k].z + w[k].w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((tid & 63) == 0) s_sum[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) out[blockIdx.x] = (s_sum[0] + s_sum[1]) + (s_sum[2] + s_sum[3]);
}

}  // namespace

extern "C" int32_t sv_read_probe(const void *buf, size_t bytes, uint32_t *out, void *stream) {
  if (!buf || !out) return 1;
  if (bytes == 0 || bytes % PCHUNK || ((uintptr_t)buf & 15) || bytes / PCHUNK > 0x7fffffffull) return 2;
  const unsigned grid = (unsigned)(bytes / PCHUNK);
  hipLaunchKernelGGL(k_read_probe, dim3(grid), dim3(PNT), 0, (hipStream_t)stream,
                     static_cast<const u32x4p *>(buf), out);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}
