// Layout adapters for the fixed-length layouts of aclnnFlashAttentionScoreV2
// ("inputLayout": BSH, SBH, BSND, BNSD), for strided (non-contiguous) TND
// tensors, and for head dims the kernels do not have (zero-padded to 64 or 128).  The attention kernels read and write
// the packed TND layout; BSH and BSND batches with one common length are
// already TND in memory, while BNSD and SBH tensors are gathered into TND
// buffers in the workspace before the kernels and the kernels' outputs are
// scattered back after them.  Pure data movement: 16 bytes per thread, the TND
// side contiguous across consecutive threads.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// Element offset of (b, s, n, 0) in a [B, S, N, D] tensor stored as `layout`
// (kLayoutStrided: a TND tensor, B = 1, with token stride ts and head stride hs).
__device__ __forceinline__ int64_t layout_row(int layout, int64_t b, int64_t s, int64_t n, int64_t B, int64_t S,
                                              int64_t N, int64_t D, int64_t ts, int64_t hs) {
  if (layout == kLayoutStrided) return s * ts + n * hs;
  if (layout == kLayoutBNSD) return ((b * N + n) * S + s) * D;
  return ((s * B + b) * N + n) * D;   // SBH
}

// TND index t = b*S + s; each thread moves one 16-byte chunk of one (t, n) row.
// The TND copy has rows of DK elements, the tensor rows of D <= DK: gathering
// fills columns D .. DK-1 with zeros, scattering moves the first D only.
__global__ __launch_bounds__(256) void fa_relayout_kernel(const char* src, char* dst, int64_t B, int64_t S,
                                                          int64_t N, int64_t D, int64_t DK, int ebytes, int layout,
                                                          int to_tnd, int64_t ts, int64_t hs) {
  const int64_t cpr = DK * ebytes / 16;   // chunks per (t, n) row of the TND copy
  const int64_t cdata = D * ebytes / 16;  // of them holding the tensor's columns
  const int64_t total = B * S * N * cpr;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t c = i % cpr;
    const int64_t row = i / cpr;         // (t, n) in TND order
    const int64_t tnd = row * DK * ebytes + 16 * c;
    if (c >= cdata) {
      if (to_tnd) *reinterpret_cast<u32x4*>(dst + tnd) = u32x4{0u, 0u, 0u, 0u};
      continue;
    }
    const int64_t n = row % N, t = row / N;
    const int64_t b = t / S, s = t - b * S;
    const int64_t lay = layout_row(layout, b, s, n, B, S, N, D, ts, hs) * ebytes + 16 * c;
    const int64_t so = to_tnd ? lay : tnd, dof = to_tnd ? tnd : lay;
    *reinterpret_cast<u32x4*>(dst + dof) = *reinterpret_cast<const u32x4*>(src + so);
  }
}

// Plan staging for calls made under stream capture: a chunk of the host-built work
// plan travels as the kernel's by-value argument (the graph keeps a copy of the
// arguments, not a pointer to host memory) and is stored to the workspace, 16 bytes
// per thread.
struct StageChunk {
  u32x4 data[kStageChunkBytes / 16];
};

__global__ __launch_bounds__(128) void fa_stage_kernel(char* dst, uint32_t n16, StageChunk c) {
  for (uint32_t x = threadIdx.x; x < n16; x += 128) reinterpret_cast<u32x4*>(dst)[x] = c.data[x];
}

hipError_t launch_stage(char* dst, const char* src, size_t bytes, hipStream_t s) {
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0) return hipErrorInvalidValue;
  for (size_t off = 0; off < bytes; off += kStageChunkBytes) {
    const size_t n = bytes - off < (size_t)kStageChunkBytes ? bytes - off : (size_t)kStageChunkBytes;
    StageChunk c;
    __builtin_memcpy(&c, src + off, n);
    hipLaunchKernelGGL(fa_stage_kernel, dim3(1), dim3(128), 0, s, dst + off, (uint32_t)(n / 16), c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_relayout(const void* src, void* dst, int64_t B, int64_t S, int64_t N, int64_t D, int64_t DK,
                           int ebytes, int layout, bool to_tnd, hipStream_t s, int64_t ts, int64_t hs) {
  if (D > DK || (D * ebytes) % 16 != 0 || (DK * ebytes) % 16 != 0) return hipErrorInvalidValue;
  if (layout != kLayoutBNSD && layout != kLayoutSBH && layout != kLayoutStrided) return hipErrorInvalidValue;
  if (layout == kLayoutStrided && B != 1) return hipErrorInvalidValue;
  const int64_t chunks = B * S * N * (DK * ebytes / 16);
  if (chunks == 0) return hipSuccess;
  const int64_t need = (chunks + 255) / 256;
  const int64_t blocks = need < 65536 ? need : 65536;
  hipLaunchKernelGGL(fa_relayout_kernel, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const char*>(src),
                     reinterpret_cast<char*>(dst), B, S, N, D, DK, ebytes, layout, to_tnd ? 1 : 0, ts, hs);
  return hipGetLastError();
}

}  // namespace fa
