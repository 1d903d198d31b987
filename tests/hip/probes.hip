// Test-only probes of gfx950 builtins whose lane layout or rounding the
// attention kernels rely on.  Each probe runs one wave over a few KB of
// caller-provided device buffers; every index stays inside them.  One more,
// probe_mfma_rate, measures the sustained matrix-core rate of the chip (a
// reference point for the attention kernels' rates, not part of any test).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// a, b: 64 lanes x 8 bf16 (raw per-lane operands); c: 64 lanes x 16 f32
__global__ void k_mfma_bf16(const bf16x8* a, const bf16x8* b, f32x16* c) {
  const int l = threadIdx.x;
  c[l] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[l], b[l], f32x16{}, 0, 0, 0);
}

// a, b: 64 lanes x 32 bytes; c: 64 lanes x 16 f32; E8M0 scales
__global__ void k_mfma_fp8(const i32x8* a, const i32x8* b, f32x16* c, int sa, int sb) {
  const int l = threadIdx.x;
  c[l] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[l], b[l], f32x16{}, 0, 0, 0, sa, 0, sb);
}

// the same with one E8M0 scale per lane for each operand (sa[l], sb[l])
__global__ void k_mfma_fp8_lanescale(const i32x8* a, const i32x8* b, f32x16* c, const int* sa, const int* sb) {
  const int l = threadIdx.x;
  c[l] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[l], b[l], f32x16{}, 0, 0, 0, sa[l], 0, sb[l]);
}

__global__ void k_mfma_fp8_unscaled(const i32x8* a, const i32x8* b, f32x16* c) {
  const int l = threadIdx.x;
  c[l] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[l], b[l], f32x16{}, 0, 0, 0, 0, 0, 0);
}

// x: 4 floats per thread -> one dword of 4 E4M3 codes (bytes in order)
__global__ void k_cvt_fp8(const float* x, uint32_t* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * i], x[4 * i + 1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * i + 2], x[4 * i + 3], w, true);
  out[i] = w;
}

// x: 64 floats -> y: 4 x 64 floats: the two results of v_permlane32_swap
// with x in both operands, then their max and their sum (the half-wave row
// max and row sum the kernels take)
__global__ void k_swap_halves(const float* x, float* y) {
  const int l = threadIdx.x;
  const unsigned u = __float_as_uint(x[l]);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  y[l] = a;
  y[64 + l] = b;
  y[128 + l] = __builtin_fmaxf(a, b);
  y[192 + l] = a + b;
}

// transposed LDS read: LDS holds u16 values 0..1023; lane l reads at byte
// offset addr[l] (caller keeps addr[l] + 8 <= 2048); out: 64 x 4 u16
__global__ void k_tr16(const int* addr, short* out) {
  __shared__ short lds[1024];
  const int l = threadIdx.x;
  for (int i = l; i < 1024; i += 64) lds[i] = (short)i;
  __syncthreads();
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) char*)lds + addr[l]));
  for (int e = 0; e < 4; ++e) out[4 * l + e] = r[e];
}

// direct-to-LDS buffer load: lane l loads the 16 bytes at byte offset
// off[l] of a buffer whose range is nbytes; LDS is then copied out (1 KB)
__global__ void k_load_lds(const uint32_t* src, const int* off, int nbytes, uint32_t* out) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[256 + 64];
  const int l = threadIdx.x;
  for (int i = l; i < 320; i += 64) lds[i] = 0xdeadbeefu;
  __syncthreads();
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds + 16), 16, off[l], 0, 0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int i = l; i < 320; i += 64) out[i] = lds[i];
}

// Sustained matrix-core rate: workgroups of 8 waves (2 per SIMD), each wave
// issuing `iters` rounds of 8 (bf16, 32x32x16) or 4 (FP8 E4M3, 32x32x64,
// unit block scales) independent products on register operands.  src: 512
// ints of operand bits; out: one float per thread (keeps the products live).
template <bool FP8>
__global__ __launch_bounds__(512) void k_mfma_rate(const int* src, float* out, int iters) {
  const int lane = threadIdx.x & 63;
  f32x16 c[8] = {};
  if constexpr (FP8) {
    i32x8 a, b;
    for (int j = 0; j < 8; ++j) {
      a[j] = src[(8 * lane + j) & 255];
      b[j] = src[256 + ((8 * lane + j) & 255)];
    }
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) c[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[k], 0, 0, 0, 127, 0, 127);
  } else {
    const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const int4*>(src + 4 * (lane & 63)));
    const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const int4*>(src + 256 + 4 * (lane & 63)));
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) r += c[k][e];
  out[blockIdx.x * 512 + threadIdx.x] = r;
}

// LDS read rate: workgroups of 8 waves, each wave issuing `iters` rounds of
// 16 reads from the first 64 KB of an LDS array: ds_read_b128 (1 KB per wave-instruction,
// consecutive 16 bytes per lane) or ds_read_b64_tr_b16 (512 bytes, the
// transposed V read of the forward kernel: 128-element rows, chunk index
// XOR (row & 3) << 2).  Every address stays inside the array.
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_t;
template <bool TR>
__global__ __launch_bounds__(512) void k_lds_rate(float* out, int iters) {
  // 96 KB so that a CU holds one workgroup (the reads use the first 64 KB)
  __shared__ __attribute__((aligned(1024))) float lds[24576];
  for (int i = threadIdx.x; i < 16384; i += 512) lds[i] = 1e-3f * (i & 1023);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, grpv = lane >> 4, sl = lane & 15;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  i16x4 acc2 = {0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
    const int sh = (it & 3) * 1024;  // floats; a new address every round
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (!TR) {
        const float4 x = *reinterpret_cast<const float4*>(&lds[((wave * 16 + r) & 15) * 256 + sh + lane * 4]);
        acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
      } else {
        const int row = (r & 3) * 16 + 4 * (wave & 1) + (sl >> 2);
        const int col = 32 * (r >> 2) + 16 * (grpv & 1) + 4 * (sl & 3);
        const int e = row * 128 + (((col >> 3) ^ ((row & 3) << 2)) << 3) + (col & 7) + 2 * sh;  // < 32768
        acc2 += __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t)(reinterpret_cast<const short*>(lds) + e));
      }
    }
  }
  out[blockIdx.x * 512 + threadIdx.x] = acc.x + acc.y + acc.z + acc.w + (float)(acc2[0] + acc2[1] + acc2[2] + acc2[3]);
}

extern "C" {
int probe_lds_rate(int tr, float* out, int iters, int grid, void* s) {
  if (tr) hipLaunchKernelGGL(k_lds_rate<true>, dim3(grid), dim3(512), 0, (hipStream_t)s, out, iters);
  else hipLaunchKernelGGL(k_lds_rate<false>, dim3(grid), dim3(512), 0, (hipStream_t)s, out, iters);
  return hipGetLastError();
}
int probe_mfma_rate(int fp8, const int* src, float* out, int iters, int grid, void* s) {
  if (fp8) hipLaunchKernelGGL(k_mfma_rate<true>, dim3(grid), dim3(512), 0, (hipStream_t)s, src, out, iters);
  else hipLaunchKernelGGL(k_mfma_rate<false>, dim3(grid), dim3(512), 0, (hipStream_t)s, src, out, iters);
  return hipGetLastError();
}
int probe_load_lds(const uint32_t* src, const int* off, int nbytes, uint32_t* out, void* s) {
  hipLaunchKernelGGL(k_load_lds, dim3(1), dim3(64), 0, (hipStream_t)s, src, off, nbytes, out);
  return hipGetLastError();
}
int probe_mfma_bf16(const void* a, const void* b, float* c, void* s) {
  hipLaunchKernelGGL(k_mfma_bf16, dim3(1), dim3(64), 0, (hipStream_t)s, (const bf16x8*)a, (const bf16x8*)b, (f32x16*)c);
  return hipGetLastError();
}
int probe_mfma_fp8(const void* a, const void* b, float* c, int sa, int sb, void* s) {
  hipLaunchKernelGGL(k_mfma_fp8, dim3(1), dim3(64), 0, (hipStream_t)s, (const i32x8*)a, (const i32x8*)b, (f32x16*)c, sa, sb);
  return hipGetLastError();
}
int probe_mfma_fp8_lanescale(const void* a, const void* b, float* c, const int* sa, const int* sb, void* s) {
  hipLaunchKernelGGL(k_mfma_fp8_lanescale, dim3(1), dim3(64), 0, (hipStream_t)s, (const i32x8*)a, (const i32x8*)b,
                     (f32x16*)c, sa, sb);
  return hipGetLastError();
}
int probe_mfma_fp8_unscaled(const void* a, const void* b, float* c, void* s) {
  hipLaunchKernelGGL(k_mfma_fp8_unscaled, dim3(1), dim3(64), 0, (hipStream_t)s, (const i32x8*)a, (const i32x8*)b, (f32x16*)c);
  return hipGetLastError();
}
int probe_cvt_fp8(const float* x, uint32_t* out, int n, void* s) {
  hipLaunchKernelGGL(k_cvt_fp8, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)s, x, out, n);
  return hipGetLastError();
}
int probe_swap_halves(const float* x, float* y, void* s) {
  hipLaunchKernelGGL(k_swap_halves, dim3(1), dim3(64), 0, (hipStream_t)s, x, y);
  return hipGetLastError();
}
int probe_tr16(const int* addr, short* out, void* s) {
  hipLaunchKernelGGL(k_tr16, dim3(1), dim3(64), 0, (hipStream_t)s, addr, out);
  return hipGetLastError();
}
}
