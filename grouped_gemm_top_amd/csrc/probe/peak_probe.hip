// peak_probe.hip -- measurement probes: dense bf16 MFMA throughput and HBM streaming
// bandwidth on gfx950 (the peaks the layer's kernels are compared against).
#include <hip/hip_runtime.h>

#include "moe_probe.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Each wavefront keeps eight (shape 0) or four (shape 1) accumulators in flight, so
// consecutive MFMAs never depend on each other and the matrix core issues back to back.
// Operands are small integers, so every sum is exact and stays far from overflow.  The MFMAs
// are written as inline assembly on VGPR operands: as builtins the compiler places these few
// accumulators in AGPRs and copies them around every iteration, which is not what a peak
// probe should time.
template <int SHAPE>
__global__ __launch_bounds__(256) void k_mfma_peak(float* __restrict__ sink, int iters) {
  const int tid = blockIdx.x * 256 + threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((threadIdx.x + i) & 3);
    b[i] = (__bf16)(float)((3 * threadIdx.x + i) & 3);
  }
  float s = 0.f;
  if constexpr (SHAPE == 0) {
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    asm volatile("s_nop 7" ::: "memory");  // the VALU writes of acc settle before the MFMAs read it
#pragma unroll 1
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[j]) : "v"(a), "v"(b));
    }
    asm volatile("s_nop 15" ::: "memory");  // the last MFMA results land before VALU reads
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  } else {
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
    asm volatile("s_nop 7" ::: "memory");
#pragma unroll 1
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc[j]) : "v"(a), "v"(b));
    }
    asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[j][v];
  }
  sink[tid] = s;
}

__global__ __launch_bounds__(256) void k_copy16(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void k_read16(const uint4* __restrict__ src, size_t n, uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t x = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    const uint4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = x;
}

// One scaled fp8 MFMA per wavefront (case c = blockIdx.x): lane L passes its 32 bytes of A
// and of B, its scale dwords (byte 0 selected) and a zero accumulator, and writes the four
// floats it receives.  Formats: e4m3 for both operands.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__global__ __launch_bounds__(64) void k_mfma_fp8_layout(const i32x8* __restrict__ a, const i32x8* __restrict__ b,
                                                        const int* __restrict__ sa, const int* __restrict__ sb,
                                                        f32x4* __restrict__ d) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  d[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], b[i], z, 0, 0, 0, sa[i], 0, sb[i]);
}

// fp32 -> fp8 e4m3 with the conversion instruction the fp8 kernels use, two values per call
__global__ __launch_bounds__(256) void k_cvt_fp8(const float* __restrict__ src, int n2, uint16_t* __restrict__ dst) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n2) dst[i] = (uint16_t)__builtin_amdgcn_cvt_pk_fp8_f32(src[2 * i], src[2 * i + 1], 0, false);
}

// Repeated reads of a buffer of `chunks` kilobytes, `passes` times over, as kilobyte loads of
// one wavefront each (wavefront v of the grid takes chunks v, v + V, ... of the pass sequence).
// mode 0: buffer_load_dwordx4 into VGPRs (eight in flight, XOR-folded into sink); mode 1:
// buffer_load_dwordx4 ... lds into a 16 KB LDS ring per wavefront with at most 12 in flight,
// the load form the GEMM kernels use; mode 2: the same with the lanes' 16-byte chunks in the
// permuted order of the GEMMs' K-strided stages (each chunk still read once).  Times the two paths from L2 (a small buffer) or HBM.
typedef int i32x4 __attribute__((ext_vector_type(4)));
template <int MODE>
__global__ __launch_bounds__(256) void k_reread(const char* __restrict__ src, uint32_t chunks, uint32_t passes,
                                                uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(1024))) char ring[4 * 16384];
  const uint32_t L = threadIdx.x & 63;
  const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t V = gridDim.x * 4, v0 = blockIdx.x * 4 + w;
  const uint64_t total = (uint64_t)chunks * passes;
  const uint64_t base = (uint64_t)src;
  const i32x4 d = {(int)(uint32_t)base, (int)((uint32_t)(base >> 32) & 0xFFFFu), (int)(chunks * 1024u), 0x00020000};
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src), (short)0,
                                                                     (int)(chunks * 1024u), 0x00020000);
  uint32_t x = 0;
  if constexpr (MODE == 0) {
    uint64_t c = v0;
    for (; c + 7 * (uint64_t)V < total; c += 8 * (uint64_t)V) {
      uint4 t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t off = (uint32_t)((c + u * (uint64_t)V) % chunks) * 1024u + L * 16u;
        t[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) x ^= t[u].x ^ t[u].y ^ t[u].z ^ t[u].w;
    }
    for (; c < total; c += V) {
      const uint4 t = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    r, (uint32_t)(c % chunks) * 1024u + L * 16u, 0, 0));
      x ^= t.x ^ t.y ^ t.z ^ t.w;
    }
  } else {
    const i32x4 ds = {__builtin_amdgcn_readfirstlane(d.x), __builtin_amdgcn_readfirstlane(d.y),
                      __builtin_amdgcn_readfirstlane(d.z), __builtin_amdgcn_readfirstlane(d.w)};
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(ring + w * 16384);
    uint32_t q = 0;
    for (uint64_t c = v0; c < total; c += V, ++q) {
      uint32_t pos = L;
      if constexpr (MODE == 2) {
        // the K-strided GEMM stage order: k-row k = 2 (q & 15) + (L >> 5) of 512 bytes, lane
        // position L & 31 holding chunk (L & 31) ^ f(k), f(k) = 2 ((k & 3) | (((k >> 3) & 1) << 2))
        const uint32_t k = 2u * (q & 15u) + (L >> 5);
        pos = (L & 32u) | ((L & 31u) ^ (2u * ((k & 3u) | (((k >> 3) & 1u) << 2))));
      }
      const uint32_t off = (uint32_t)(c % chunks) * 1024u + pos * 16u;
      asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds\n\ts_waitcnt vmcnt(12)"
                   ::"v"(off), "s"(ds), "{m0}"(m0 + (q & 15u) * 1024u) : "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = x;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" int moe_probe_mfma_bf16(int shape, int blocks, int iters, float* sink, void* stream) {
  if (sink == nullptr || (shape != 0 && shape != 1) || blocks < 1 || blocks > 65536 || iters < 1 ||
      iters > (1 << 24))
    return 1;
  hipStream_t s = (hipStream_t)stream;
  if (shape == 0) hipLaunchKernelGGL(k_mfma_peak<0>, dim3(blocks), dim3(256), 0, s, sink, iters);
  else hipLaunchKernelGGL(k_mfma_peak<1>, dim3(blocks), dim3(256), 0, s, sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int moe_probe_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (src == nullptr || dst == nullptr || bytes % 16 != 0 || !aligned16(src) || !aligned16(dst) || blocks < 1 ||
      blocks > 65536)
    return 1;
  if (bytes == 0) return 0;
  hipLaunchKernelGGL(k_copy16, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)src, (uint4*)dst,
                     bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int moe_probe_read(const void* src, size_t bytes, int blocks, uint32_t* sink, void* stream) {
  if (src == nullptr || sink == nullptr || bytes % 16 != 0 || !aligned16(src) || blocks < 1 || blocks > 65536)
    return 1;
  if (bytes == 0) return 0;
  hipLaunchKernelGGL(k_read16, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4*)src, bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int moe_probe_mfma_fp8_layout(const uint8_t* a, const uint8_t* b, const uint32_t* sa, const uint32_t* sb,
                                         int cases, float* d, void* stream) {
  if (!a || !b || !sa || !sb || !d || cases < 1 || cases > 4096 || !aligned16(a) || !aligned16(b) || !aligned16(d))
    return 1;
  hipLaunchKernelGGL(k_mfma_fp8_layout, dim3(cases), dim3(64), 0, (hipStream_t)stream, (const i32x8*)a,
                     (const i32x8*)b, (const int*)sa, (const int*)sb, (f32x4*)d);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int moe_probe_cvt_fp8(const float* src, int n, uint8_t* dst, void* stream) {
  if (!src || !dst || n < 2 || n % 2 != 0 || ((uintptr_t)dst & 1u)) return 1;
  const int n2 = n / 2;
  hipLaunchKernelGGL(k_cvt_fp8, dim3((n2 + 255) / 256), dim3(256), 0, (hipStream_t)stream, src, n2, (uint16_t*)dst);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int moe_probe_reread(const void* src, size_t bytes, int passes, int mode, int blocks, uint32_t* sink,
                                void* stream) {
  if (!src || !sink || !aligned16(src) || bytes < 1024 || bytes % 1024 != 0 || bytes > ((size_t)1 << 30) ||
      passes < 1 || passes > 4096 || mode < 0 || mode > 2 || blocks < 1 || blocks > 65536)
    return 1;
  const uint32_t chunks = (uint32_t)(bytes / 1024);
  if (mode == 0)
    hipLaunchKernelGGL(k_reread<0>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const char*)src, chunks,
                       (uint32_t)passes, sink);
  else if (mode == 1)
    hipLaunchKernelGGL(k_reread<1>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const char*)src, chunks,
                       (uint32_t)passes, sink);
  else
    hipLaunchKernelGGL(k_reread<2>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const char*)src, chunks,
                       (uint32_t)passes, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
