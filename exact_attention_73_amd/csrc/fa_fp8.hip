// FP8 E4M3 path for gfx950: the prep kernel (rotation, block scales,
// quantisation, V transpose) and the FP8 attention forward.
//
// Prep (FA3 explainer "FlashAttention-3：用异步流水榨出 Hopper 的 Attention 性能",
// sections "Block Quantization 为什么优于 Per-Tensor Scale" and "Incoherent
// Processing 如何摊平离群值"; E4M3 largest value 448 from the wmrh.cn
// FlashAttention V3 article, section 三.3):
//   y = x diag(sigma_h) H_d (unnormalised fast Walsh-Hadamard transform,
//       log2(d) butterfly stages: 3 inside a lane, 4 across 16 lanes),
//   a = max |y| over each 128-row block, codes = RNE(y * 448 / a),
//   stored scale s = a / (448 sqrt(d)) for rotated tensors (the 1/sqrt(d)
//   of the orthonormal rotation is folded into s), a / 448 otherwise.
// One workgroup per (batch, head, 128-row block); HBM-bound: it reads the
// bf16 tensor once and writes the codes once.  V is written transposed,
// [d][ld], through an LDS transpose, so the forward kernel's PV operand is
// key-contiguous ("FP8 路径的第一个问题：WGMMA Layout" section: the transpose is
// fused into a pass that happens anyway instead of costing its own HBM
// round trip).
//
// Forward: same decomposition, data path and online softmax as the bf16
// kernel (one workgroup of 4 waves per 128 query rows, direct-to-LDS K and
// V^T rings with K one tile ahead, S^T = K Q^T and O^T = V^T P^T on
// v_mfma_f32_32x32x64_f8f6f4 with fp32 accumulation and softmax state).
// The exponent reference of P is the running max rounded up to a whole
// number in the log2 domain, so P is in (0, 1] and every change of
// reference is an exact power of two: O and l are accumulated against the
// first tile's reference and each tile's P^T enters the PV product scaled
// by 2^(reference - base) through the instruction's per-lane E8M0 scale of
// the B operand, so O is never rescaled.  Scores are descaled by folding
// s_Q,i * s_K,j into the exp2 constant of each tile; probabilities are
// produced directly as P * 2^7 * mu_j (exp2 bias) and cast to E4M3, and the
// PV instruction's block exponents supply 2^-7 (P, times the shift) and
// 2^e_j (V), where s_V,j = mu_j * 2^e_j.  Non-causal batches of 1024 or
// more rows and causal ones of 4096 or more run fwd_fp8_pp_kernel instead:
// the same arithmetic with eight waves per workgroup in two groups that take
// turns on each SIMD's matrix core (ping-pong).  Shorter causal batches run
// the four-wave kernel with one S buffer per wave at three workgroups per CU.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr float kE4M3Max = 448.f;

// ---------------------------------------------------------------------------
// prep
// ---------------------------------------------------------------------------
enum PrepMode { kPrepFused = 0, kPrepAmaxOnly = 1, kPrepGlobalScale = 2 };

// Four floats to E4M3 (round to nearest even), packed low to high.  The
// first conversion writes bytes 0-1 and keeps the upper half of its `old`
// operand, which the second conversion then overwrites, so `old` may be
// any value: a's own bits, whose register is free after this conversion,
// spare a zero initialisation.
__device__ __forceinline__ uint32_t cvt_e4m3x4(float a, float b, float c, float d) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_uint(a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

__device__ __forceinline__ float clamp_e4m3(float x) { return __builtin_fminf(__builtin_fmaxf(x, -kE4M3Max), kE4M3Max); }

// Value of lane L ^ B (B in 1, 2, 4, 8, inside each row of 16 lanes) through
// DPP lane moves: quad_perm [1,0,3,2] and [2,3,0,1] give ^1 and ^2; ^4 is
// row_half_mirror (^7) then quad_perm [3,2,1,0] (^3); ^8 is row_mirror (^15)
// then row_half_mirror (^7).
template <int DPP> __device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), DPP, 0xf, 0xf, true));
}
template <int B> __device__ __forceinline__ float lane_xor16(float x) {
  if constexpr (B == 1) return dpp_mov<0xB1>(x);
  else if constexpr (B == 2) return dpp_mov<0x4E>(x);
  else if constexpr (B == 4) return dpp_mov<0x1B>(dpp_mov<0x141>(x));
  else return dpp_mov<0x141>(dpp_mov<0x140>(x));
}

// One workgroup = 256 threads = 16 row groups x 16 lanes; a lane owns 8
// consecutive d of 8 consecutive rows (row = 8 * group + it).
template <int MODE>
__global__ __launch_bounds__(256) void fp8_prep_kernel(Fp8PrepParams p) {
  constexpr int D = 128;
  __shared__ float red[4];
  // transposed codes, one row of 128 keys per d as 32 words plus one pad
  // word: the odd row stride spreads both the column writes and the row
  // gathers below over the LDS banks
  __shared__ uint32_t tr[D][33];

  const int nb = (p.N + 127) / 128;
  const int blk = blockIdx.x % nb;
  const int bh = blockIdx.x / nb;
  const int h = bh % p.H;
  const int tid = threadIdx.x, lr = tid & 15, grp = tid >> 4;
  const int n0 = blk * 128;
  const uint16_t* X = p.x + (size_t)bh * p.N * D;
  const bool rot = p.signs != nullptr;

  float sgn[4];  // +1 in the lower lane of each butterfly pair, -1 in the upper
#pragma unroll
  for (int i = 0; i < 4; ++i) sgn[i] = (lr >> i) & 1 ? -1.f : 1.f;
  float sg[8];
  if (rot) {
    const int8_t* s8 = p.signs + h * D + lr * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) sg[e] = (float)s8[e];
  }

  // All eight rows are requested before any arithmetic: buffer loads with a
  // range of N rows, so rows past N read as zero without a branch (a branch
  // per row made each load wait for the previous one).  Input and codes are
  // each touched once, so loads and stores use the non-temporal cache
  // policy (cache-policy bit 1); measured with cold caches this moves Q
  // from 2.7 to 3.7 TB/s and the transposed V from 2.9 to 4.5 TB/s.
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X), 0, p.N * D * 2, 0x00020000);
  u32x4 raw[8];
#pragma unroll
  for (int it = 0; it < 8; ++it)
    raw[it] = __builtin_amdgcn_raw_buffer_load_b128(rx, ((n0 + grp * 8 + it) * D + lr * 8) * 2, 0, 2);

  float y[8][8];
  float amax = 0.f;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[it][2 * e] = __uint_as_float(raw[it][e] << 16);
      y[it][2 * e + 1] = __uint_as_float(raw[it][e] & 0xffff0000u);
    }
    if (rot) {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[it][e] *= sg[e];
      // butterflies over index bits 0..2 (inside the lane)
#pragma unroll
      for (int b = 1; b < 8; b <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (!(e & b)) {
            const float u = y[it][e], w = y[it][e + b];
            y[it][e] = u + w;
            y[it][e + b] = u - w;
          }
      // butterflies over index bits 3..6 (lanes lr ^ 1, 2, 4, 8 of the row):
      // the lower lane keeps y + o, the upper one o - y, i.e. o + sgn * y
#pragma unroll
      for (int e = 0; e < 8; ++e) y[it][e] = lane_xor16<1>(y[it][e]) + sgn[0] * y[it][e];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[it][e] = lane_xor16<2>(y[it][e]) + sgn[1] * y[it][e];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[it][e] = lane_xor16<4>(y[it][e]) + sgn[2] * y[it][e];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[it][e] = lane_xor16<8>(y[it][e]) + sgn[3] * y[it][e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(y[it][e]));
  }

  const float norm = rot ? 11.313708498984761f : 1.f;  // sqrt(128)
  if (MODE == kPrepGlobalScale) {
    // the tensor's amax = max over every block amax left by the first pass
    amax = 0.f;
    const int n = (int)gridDim.x;
    for (int i = tid; i < n; i += 256) amax = __builtin_fmaxf(amax, p.scale[i]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  if (MODE == kPrepAmaxOnly) {
    if (tid == 0) p.scale[blockIdx.x] = amax;  // raw block amax of y; the scales are written last
    return;
  }
  // multiplier turning y into the E4M3 range; the same expression in both modes
  float inv, s_out;
  if (p.pow2) {
    // s = 2^k, k = ceil(log2(amax / 448)) from the bits of amax (448 = 1.75 * 2^8)
    const uint32_t ab = __float_as_uint(amax);
    int k = (int)((ab >> 23) & 0xffu) - 127 - 8 + ((ab & 0x7fffffu) > 0x600000u ? 1 : 0);
    k = max(k, -126);
    s_out = amax > 0.f ? __uint_as_float((uint32_t)(k + 127) << 23) : 1.f;
    inv = amax > 0.f ? __uint_as_float((uint32_t)(127 - k) << 23) : 0.f;  // exact 2^-k
  } else {
    s_out = amax > 0.f ? amax / (kE4M3Max * norm) : 1.f;
    inv = amax > 0.f ? kE4M3Max / amax : 0.f;
  }
  if (MODE == kPrepFused && tid == 0) p.scale[blockIdx.x] = s_out;

  if (!p.transpose) {
    // codes through range-checked buffer stores: rows past N are dropped
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(p.x8 + (size_t)bh * p.N * D, 0, p.N * D, 0x00020000);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int n = n0 + grp * 8 + it;
      u32x2 w;
      w[0] = cvt_e4m3x4(clamp_e4m3(y[it][0] * inv), clamp_e4m3(y[it][1] * inv), clamp_e4m3(y[it][2] * inv),
                        clamp_e4m3(y[it][3] * inv));
      w[1] = cvt_e4m3x4(clamp_e4m3(y[it][4] * inv), clamp_e4m3(y[it][5] * inv), clamp_e4m3(y[it][6] * inv),
                        clamp_e4m3(y[it][7] * inv));
      __builtin_amdgcn_raw_buffer_store_b64(w, ry, n * D + lr * 8, 0, 2);
    }
  } else {
    // codes of d = 8 lr + e, rows 8 grp .. 8 grp + 7 -> words 2 grp, 2 grp + 1 of tr[d]
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u32x2 w;
      w[0] = cvt_e4m3x4(clamp_e4m3(y[0][e] * inv), clamp_e4m3(y[1][e] * inv), clamp_e4m3(y[2][e] * inv),
                        clamp_e4m3(y[3][e] * inv));
      w[1] = cvt_e4m3x4(clamp_e4m3(y[4][e] * inv), clamp_e4m3(y[5][e] * inv), clamp_e4m3(y[6][e] * inv),
                        clamp_e4m3(y[7][e] * inv));
      tr[lr * 8 + e][grp * 2] = w[0];
      tr[lr * 8 + e][grp * 2 + 1] = w[1];
    }
    __syncthreads();
    // Row d of the block: 128 keys = two 64-key segments of 16 four-key
    // groups each.  Within a segment, word w of the output holds key group
    // 2 (w % 8) + w / 8 (even groups first, then odd groups): the order in
    // which a lane of the forward kernel's PV product takes its keys.
    uint8_t* Y = p.x8 + (size_t)bh * D * p.ld;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = tid + 256 * i, d = ci >> 3, ch = ci & 7;
      const int seg = ch >> 2, w0 = (ch & 3) * 4;
      const uint32_t* row = &tr[d][0];
      u32x4 v;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int w = w0 + t;
        v[t] = row[16 * seg + 2 * (w & 7) + (w >> 3)];
      }
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(Y + (size_t)d * p.ld + n0 + ch * 16));
    }
  }
}

// Global amax over all block amaxes -> one scale written to every entry
// (runs after the quantising pass, which reads the block amaxes).
__global__ __launch_bounds__(1024) void fp8_tensor_scale_kernel(float* scale, int n, float norm, bool pow2) {
  __shared__ float red[16];
  float a = 0.f;
  for (int i = threadIdx.x; i < n; i += 1024) a = __builtin_fmaxf(a, scale[i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = __builtin_fmaxf(a, red[i]);
  float s = a > 0.f ? a / (kE4M3Max * norm) : 1.f;
  if (pow2 && a > 0.f) {
    const uint32_t ab = __float_as_uint(a);
    const int k = max((int)((ab >> 23) & 0xffu) - 127 - 8 + ((ab & 0x7fffffu) > 0x600000u ? 1 : 0), -126);
    s = __uint_as_float((uint32_t)(k + 127) << 23);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += 1024) scale[i] = s;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
constexpr int kWaves = 4;
constexpr int kQW = 32;
constexpr int kBR = kWaves * kQW;  // 128 = one scale block of queries
constexpr int kBC = 64;            // keys per tile (half a scale block)
constexpr int kPPKeys = 128;       // keys per tile of the ping-pong kernel (one scale block)
constexpr int kThreads = kWaves * 64;

typedef __attribute__((address_space(3))) void* lds_void_t;

// vmcnt(0), expcnt and lgkmcnt left open; as a builtin the compiler knows the
// vector-memory counter is empty afterwards and adds no waits of its own
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 16 bytes per lane from buffer offset voff straight into LDS at dst + 16 * lane
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint8_t* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t)dst, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// 16-byte chunk swizzles: K rows are 128 bytes (two rows per 256 bytes of
// banks), V^T tile rows are 64 bytes (four rows per 256 bytes); the
// ping-pong kernel's 128-key V^T tile rows are 128 bytes and take the K one.
__device__ __forceinline__ int k8_swizzle(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int v8_swizzle(int d) { return (d >> 2) & 3; }

// Causal batches below the ping-pong kernel's length run this kernel with
// one S buffer per wave and three workgroups per CU (166-168 VGPRs): a step
// computes S_j, its softmax and its PV product in turn and the three waves
// of a SIMD overlap each other's matrix and vector work; the vector unit,
// which bounds the FP8 step, then has a third wave to fill its gaps (same-box
// runs of 30-60 launches: 1.05-1.07 x over two workgroups with the S double
// buffer at N = 1024-2048).  Non-causal batches keep the double buffer (with
// one buffer the compiler spills hoisted LDS addresses there).
template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, CAUSAL ? 3 : 2) void fwd_fp8_kernel(FwdFp8Params p) {
  constexpr int D = 128;
  constexpr bool ONE_S = CAUSAL;  // one S buffer per wave
  constexpr int NKB = kBC / 32;  // 2 key blocks of S^T per tile
  constexpr int NDB = D / 32;    // 4
  constexpr int NQS = D / 64;    // 2 k-steps of 64 d
  constexpr int TILE = kBC * D;  // bytes of a K tile (and of a V^T tile)
  constexpr int IPW = TILE / 1024 / kWaves;  // 1 KB wave-loads per wave per tile (2)

  // one LDS object per ring slot (compile-time slots: see the bf16 kernel)
  __shared__ __attribute__((aligned(1024))) uint8_t Ks0[TILE];  // [key][d], swizzled
  __shared__ __attribute__((aligned(1024))) uint8_t Ks1[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t Vs0[TILE];  // [d][64 keys], swizzled
  __shared__ __attribute__((aligned(1024))) uint8_t Vs1[TILE];

  const int N = p.N;
  const int BH = p.B * p.H;
  const int nq = (N + kBR - 1) / kBR;
  const int nb = nq;  // scale blocks per head (128 rows)
  int bh, qt;
  if constexpr (CAUSAL) {
    qt = nq - 1 - (int)blockIdx.x / BH;
    bh = (int)blockIdx.x % BH;
  } else {
    const int w = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
    bh = w / nq;
    qt = w % nq;
  }

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const uint8_t* __restrict__ Qg = p.q8 + (size_t)bh * N * D;
  const float* __restrict__ ks = p.ks + (size_t)bh * nb;
  const float* __restrict__ vs = p.vs + (size_t)bh * nb;
  const int q0 = qt * kBR + wave * kQW;
  const int qrow = q0 + l32;
  const float cq = p.c * p.qs[(size_t)bh * nb + qt];

  // Q^T operand: k-step s holds d = 64 s + 32 hi .. +31 of row qrow
  i32x8 qreg[NQS];
  {
    const bool ok = qrow < N;
    const u32x4* src = reinterpret_cast<const u32x4*>(Qg + (size_t)(ok ? qrow : 0) * D);
#pragma unroll
    for (int s = 0; s < NQS; ++s) {
      const u32x4 a = ok ? src[4 * s + 2 * hi] : u32x4{0, 0, 0, 0};
      const u32x4 b = ok ? src[4 * s + 2 * hi + 1] : u32x4{0, 0, 0, 0};
      qreg[s] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    }
  }

  const int kend = CAUSAL ? min(N, qt * kBR + kBR) : N;
  const int ntiles = (kend + kBC - 1) / kBC;

  // ---- direct-to-LDS loads -------------------------------------------------
  // K: wave-load i of wave w fills 8 rows of 128 bytes; lane L writes
  // physical chunk L % 8 of row L / 8.  V^T: wave-load i fills 16 rows (d) of
  // 64 bytes (the tile's keys of that row); lane L writes physical chunk
  // L % 4 of row L / 4.  Each lane fetches the logical chunk the swizzle
  // puts there.  The V^T rows arrive already in the PV operand's key order.
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(p.k8 + (size_t)bh * N * D, N * D);
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(p.v8t + (size_t)bh * D * p.ld, D * p.ld);
  int koff[IPW], voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int ins = wave * IPW + i;
    const int kr = ins * 8 + (lane >> 3), kc = lane & 7;
    koff[i] = kr * D + ((kc ^ k8_swizzle(kr)) * 16);
    const int vd = ins * 16 + (lane >> 2), vc = lane & 3;
    voff[i] = vd * p.ld + ((vc ^ v8_swizzle(vd)) * 16);
  }
  auto issue_k = [&](uint8_t* dst, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) lds_dma16(rk, dst + (wave * IPW + i) * 1024, koff[i] + j * kBC * D);
  };
  auto issue_v = [&](uint8_t* dst, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) lds_dma16(rv, dst + (wave * IPW + i) * 1024, voff[i] + j * kBC);
  };

  auto qk = [&](f32x16 (&s)[NKB], const uint8_t* kt) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int st = 0; st < NQS; ++st)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int row = kb * 32 + l32;
        const uint8_t* krow = kt + row * D;
        const int sw = k8_swizzle(row);
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(krow + (((4 * st + 2 * hi) ^ sw) * 16));
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(krow + (((4 * st + 2 * hi + 1) ^ sw) * 16));
        const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                         (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        s[kb] = mfma_fp8_32x32x64(a, qreg[st], s[kb], 127, 127);
      }
  };

  float ks_next = 0.f, vs_next = 0.f;  // K and V scales of the next tile to process
  // P's exponent reference: the running max of the log2-domain scores of row
  // qrow rounded up to a whole number (P = 2^(t - m_ref) in (0, 1]).  O and l
  // are accumulated against m_base, the reference of the first tile; each
  // tile's P^T enters the PV product scaled by 2^(m_ref - m_base), exactly,
  // through the instruction's per-lane E8M0 scale of the B operand (both
  // half-waves of a query row carry the same value), so O is never rescaled.
  float m_ref = -INFINITY;
  float m_base = 0.f;
  float l_run = 0.f;
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};

  // one step for tile j: softmax of S_j (s_in), S_{j+1} into s_out,
  // O += V_j^T P_j^T; ring slots as in the bf16 kernel.
  // raw row max (before the scale) of one S^T tile: in-lane, then with the other half wave
  auto rowmax = [&](const f32x16 (&sv)[NKB]) __attribute__((always_inline)) -> float {
    float m = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) m = fmax3(m, sv[kb][r], sv[kb][r + 1]);
    return max_halves(m);
  };

  // mx: raw row max of s_in on entry, of s_out on exit (taken at the end of
  // the step so that the S_{j+1} products stay in this step's block)
  // With ONE_S, K_j and V_j sit in slot j % 2 and the step requests K_{j+1}
  // and V_{j+1} into the other slot (read by the previous step, which every
  // wave has left at the barrier), then computes S_j itself; k_this is then
  // the tile of this step and k_next the slot to fill.
  auto step = [&](int j, f32x16 (&s_in)[NKB], f32x16 (&s_out)[NKB], float& mx, uint8_t* k_this,
                  uint8_t* k_next, const uint8_t* v_this, uint8_t* v_next) __attribute__((always_inline)) {
    const int key0 = j * kBC;
    wait_vmem_all();
    __syncthreads();
    // the scales of tile j arrived with the previous step's loads; fetch
    // those of tile j + 1 behind this step's DMAs
    const float ksc = ks_next, vsc = vs_next;
    if constexpr (ONE_S) {
      if (j + 1 < ntiles) issue_k(k_next, j + 1);
    } else {
      if (j + 2 < ntiles) issue_k(k_this, j + 2);
    }
    if (j + 1 < ntiles) {
      issue_v(v_next, j + 1);
      ks_next = ks[(key0 + kBC) >> 7];
      vs_next = vs[(key0 + kBC) >> 7];
    }
    if (CAUSAL && key0 > q0 + kQW - 1) return;
    if constexpr (ONE_S) {
      qk(s_in, k_this);
      mx = rowmax(s_in);
    }

    const float ct = cq * ksc;
    const uint32_t svb = __float_as_uint(vsc);
    const int v_exp = (int)((svb >> 23) & 0xffu);                          // E8M0 exponent of s_V
    const float mu = __uint_as_float((svb & 0x007fffffu) | 0x3f800000u);  // s_V mantissa in [1, 2)
    const float pbias = 7.f + __builtin_amdgcn_logf(mu);                  // log2(2^7 mu); 7 for power-of-two s_V
    const float inv_f = __builtin_amdgcn_rcpf(128.f * mu);  // exact for the power-of-two V scales

    const bool need_mask = (CAUSAL && key0 + kBC - 1 > q0) || (key0 + kBC > N);
    if (need_mask) {
      // key = key0 + 4 hi + off, off a constant per register: the key is past
      // the row (causal) or past N iff off > lim
      int lim = N - 1 - key0 - 4 * hi;
      if constexpr (CAUSAL) lim = min(lim, qrow - key0 - 4 * hi);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
          s_in[kb][r] = off > lim ? -INFINITY : s_in[kb][r];
        }
      mx = rowmax(s_in);
    }
    m_ref = __builtin_fmaxf(m_ref, __builtin_ceilf(mx * ct));  // ct > 0; -inf stays -inf
    // every row sees key 0 in tile 0, so its reference is finite from there on
    if (j == 0) m_base = (m_ref == -INFINITY) ? 0.f : m_ref;
    float shift = (m_ref == -INFINITY) ? 0.f : m_ref - m_base;  // a whole number >= 0
    const float moff = ((m_ref == -INFINITY) ? 0.f : m_ref) - pbias;

    if constexpr (!ONE_S) qk(s_out, k_next);  // S_{j+1}: matrix cores, while the exps below run
    i32x8 pb;
    float ls[4] = {-0.f, -0.f, -0.f, -0.f};  // x + -0 = x: the first adds fold away
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, r = 4 * (w & 3);
      const float e0 = exp2_fast(__builtin_fmaf(s_in[kb][r], ct, -moff));  // P * 2^7 * mu
      const float e1 = exp2_fast(__builtin_fmaf(s_in[kb][r + 1], ct, -moff));
      const float e2 = exp2_fast(__builtin_fmaf(s_in[kb][r + 2], ct, -moff));
      const float e3 = exp2_fast(__builtin_fmaf(s_in[kb][r + 3], ct, -moff));
      ls[w & 3] += (e0 + e1) + (e2 + e3);
      pb[w] = (int)cvt_e4m3x4(e0, e1, e2, e3);
    }
    const float lsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
    // The test also reads lsum and (with two S buffers) the last S_{j+1}
    // product (finite scores: adding 0 * s is exact), which keeps the
    // products and the softmax in one block ahead of the branch, where the
    // compiler interleaves them.
    const float s_dep = ONE_S ? 0.f : 0.f * (s_out[0][15] + s_out[NKB - 1][15]);
    if (__any(shift + s_dep > 64.f && lsum >= 0.f)) {
      // rare (scores grew by more than 2^64 over the first tile's): move the
      // base so O and l stay far from the fp32 range; an exact power of two
      const float f = exp2_fast(-shift);
      l_run *= f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= f;
      m_base += shift;
      shift = 0.f;
    }
    const int ishift = (int)shift;
    l_run += lsum * __builtin_amdgcn_ldexpf(inv_f, ishift);
    // O^T += V^T P^T: lane half hi reads the 32 bytes [32 hi, 32 hi + 32) of
    // row d, which hold keys 8w + 4hi .. +3 for w = 0..7 (the prep's order)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 32 + l32;
      const uint8_t* vrow = v_this + d * kBC;
      const int sw = v8_swizzle(d);
      const u32x4 c0 = *reinterpret_cast<const u32x4*>(vrow + (((2 * hi) ^ sw) * 16));
      const u32x4 c1 = *reinterpret_cast<const u32x4*>(vrow + (((2 * hi + 1) ^ sw) * 16));
      const i32x8 a = {(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3],
                       (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
      o[db] = mfma_fp8_32x32x64(a, pb, o[db], v_exp, 127 - 7 + ishift);
    }
    if constexpr (!ONE_S) mx = rowmax(s_out);
  };

  float mx = -INFINITY;
  issue_k(Ks0, 0);
  issue_v(Vs0, 0);
  ks_next = ks[0];
  vs_next = vs[0];
  if constexpr (ONE_S) {
    f32x16 sa[NKB];
    for (int j = 0; j < ntiles; j += 2) {
      step(j, sa, sa, mx, Ks0, Ks1, Vs0, Vs1);
      if (j + 1 < ntiles) step(j + 1, sa, sa, mx, Ks1, Ks0, Vs1, Vs0);
    }
  } else {
    f32x16 sa[NKB], sb[NKB];
    if (ntiles > 1) issue_k(Ks1, 1);
    wait_vmem_all();
    __syncthreads();
    qk(sa, Ks0);
    mx = rowmax(sa);
    for (int j = 0; j < ntiles; j += 2) {
      step(j, sa, sb, mx, Ks0, Ks1, Vs0, Vs1);
      if (j + 1 < ntiles) step(j + 1, sb, sa, mx, Ks1, Ks0, Vs1, Vs0);
    }
  }

  const float l_tot = sum_halves(l_run);
  if (qrow < N) {
    const float inv = 1.f / l_tot;
    float* orow = p.o + (size_t)bh * N * D + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 val = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                           o[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * g + 4 * hi) = val;
      }
    if (hi == 0) p.lse[(size_t)bh * N + qrow] = m_base * 0.6931471805599453f + __logf(l_tot);
  }
}

// FP8 forward with the matrix/vector ping-pong of the bf16 d = 128 kernel
// (FA3 explainer, section "第二层重叠：Ping-Pong Scheduling"): eight waves per
// workgroup (256 query rows, two 128-row Q scale blocks), waves w and w + 4
// on one SIMD.  Its tiles are 128 keys, one K and V scale block each (the
// four-wave kernel's are 64): an FP8 product does the work of four bf16 ones
// in twice the cycles, so 128-key tiles give each slot as many matrix cycles
// as the bf16 kernel's 64-key slots and halve the barriers per key (measured
// 1.05-1.11 x over 64-key tiles).  The exponent reference therefore moves
// once per 128 keys (fa_fp8_ref_block).  A tile's step splits into a matrix
// part (S_t = K_t Q^T: 8 products; O^T += V_{t-1}^T P_{t-1}^T: 8 products with
// the per-lane E8M0 scales, two per 32 rows of d, one per 64-key half) and a
// vector part (the FP8 softmax of S_t: mask, power-of-two exponent
// reference, E4M3 P, fp32 row sum, rare rebase).  In every slot one group
// runs matrix parts while the other runs vector parts; group 1 runs the same
// sequence one slot later.  Stage t = {K_t, V_{t-1}^T} (32 KB) is requested
// by group 0 at the start of its matrix part of stage t - 1.
template <bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fwd_fp8_pp_kernel(FwdFp8Params p) {
  constexpr int D = 128, NW = 8, BR = NW * kQW;
  constexpr int KT = kPPKeys;            // keys per tile
  constexpr int NKB = KT / 32, NDB = D / 32, NQS = D / 64, NSUB = KT / 64;
  constexpr int TILE = KT * D;           // bytes of a K tile (and of a V^T tile)
  constexpr int IPL = TILE / 1024 / 4;   // 1 KB wave-loads per loading wave and tile
  constexpr int CPR = KT / 16;           // 16-byte chunks per V^T tile row

  __shared__ __attribute__((aligned(1024))) uint8_t Ks0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t Ks1[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t Vs0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t Vs1[TILE];

  const int N = p.N;
  const int BH = p.B * p.H;
  const int nq = (N + BR - 1) / BR;
  const int nb = (N + 127) / 128;  // scale blocks per head
  int bh, qt;
  if constexpr (CAUSAL) {
    causal_order(BH, nq, bh, qt);
  } else {
    const int w = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
    bh = w / nq;
    qt = w % nq;
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int grp = wave >> 2;
  const uint8_t* __restrict__ Qg = p.q8 + (size_t)bh * N * D;
  const float* __restrict__ ks = p.ks + (size_t)bh * nb;
  const float* __restrict__ vs = p.vs + (size_t)bh * nb;
  const int q0 = qt * BR + wave * kQW;
  const int qrow = q0 + l32;
  const float cq = p.c * p.qs[(size_t)bh * nb + min(q0 >> 7, nb - 1)];  // this wave's Q scale block

  // Q^T operand (k-step s: d = 64 s + 32 hi .. +31 of row qrow) through
  // range-checked buffer loads, ahead of the tile requests
  i32x8 qreg[NQS];
  {
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(Qg, N * D);
#pragma unroll
    for (int st = 0; st < NQS; ++st) {
      const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, qrow * D + (4 * st + 2 * hi) * 16, 0, 0));
      const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, qrow * D + (4 * st + 2 * hi + 1) * 16, 0, 0));
      qreg[st] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  const int kend = CAUSAL ? min(N, qt * BR + BR) : N;
  const int T = (kend + KT - 1) / KT;                                     // tiles of the workgroup
  const int Tw = CAUSAL ? min(T, (q0 + kQW - 1) / KT + 1) : T;            // tiles this wave uses

  // group 0 loads each stage: K rows and V^T tile rows of 128 bytes, with
  // the same chunk swizzle
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(p.k8 + (size_t)bh * N * D, N * D);
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(p.v8t + (size_t)bh * D * p.ld, D * p.ld);
  const int lw = wave & 3;
  int koff[IPL], voff[IPL];
#pragma unroll
  for (int i = 0; i < IPL; ++i) {
    const int ins = lw * IPL + i;
    const int kr = ins * 8 + (lane >> 3), kc = lane & 7;
    koff[i] = kr * D + ((kc ^ k8_swizzle(kr)) * 16);
    const int vd = ins * (64 / CPR) + lane / CPR, vc = lane % CPR;
    voff[i] = vd * p.ld + ((vc ^ k8_swizzle(vd)) * 16);
  }
  auto issue_k = [&](uint8_t* dst, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < IPL; ++i) lds_dma16(rk, dst + (lw * IPL + i) * 1024, koff[i] + j * KT * D);
  };
  auto issue_v = [&](uint8_t* dst, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < IPL; ++i) lds_dma16(rv, dst + (lw * IPL + i) * 1024, voff[i] + j * KT);
  };

  // running state: see fwd_fp8_kernel (power-of-two exponent reference
  // m_ref, accumulation base m_base, O never rescaled except on a rebase)
  float m_ref = -INFINITY, m_base = 0.f, l_run = 0.f;
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  f32x16 sc[NKB];
  i32x8 pb[NSUB];         // E4M3 P^T of the last vector part, per 64-key half (B operands of the next PV)
  int ishift = 0, v_exp = 127;

  auto mfma_part = [&](int t, const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) {
    if (t < Tw) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sc[kb] = f32x16{};
#pragma unroll
      for (int st = 0; st < NQS; ++st)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int row = kb * 32 + l32;
          const uint8_t* krow = kt + row * D;
          const int sw = k8_swizzle(row);
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(krow + (((4 * st + 2 * hi) ^ sw) * 16));
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(krow + (((4 * st + 2 * hi + 1) ^ sw) * 16));
          const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                           (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          sc[kb] = mfma_fp8_32x32x64(a, qreg[st], sc[kb], 127, 127);
        }
    }
    if (t >= 1 && t <= Tw) {
      // half sub of the tile: lane half hi reads the 32 bytes [64 sub + 32 hi,
      // +32) of row d, keys 64 sub + 8w + 4hi .. +3 for w = 0..7 (the prep's
      // order within each aligned run of 64 keys)
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int d = db * 32 + l32;
          const uint8_t* vrow = vt + d * KT;
          const int sw = k8_swizzle(d);
          const u32x4 c0 = *reinterpret_cast<const u32x4*>(vrow + (((4 * sub + 2 * hi) ^ sw) * 16));
          const u32x4 c1 = *reinterpret_cast<const u32x4*>(vrow + (((4 * sub + 2 * hi + 1) ^ sw) * 16));
          const i32x8 a = {(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3],
                           (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
          o[db] = mfma_fp8_32x32x64(a, pb[sub], o[db], v_exp, 127 - 7 + ishift);
        }
    }
  };

  auto vector_part = [&](int t, float ksc, float vsc) __attribute__((always_inline)) {
    if (t >= Tw) return;
    const int key0 = t * KT;
    const float ct = cq * ksc;
    const uint32_t svb = __float_as_uint(vsc);
    const int vexp_t = (int)((svb >> 23) & 0xffu);                        // E8M0 exponent of s_V
    const float mu = __uint_as_float((svb & 0x007fffffu) | 0x3f800000u);  // s_V mantissa in [1, 2)
    const float pbias = 7.f + __builtin_amdgcn_logf(mu);
    const float inv_f = __builtin_amdgcn_rcpf(128.f * mu);
    if ((CAUSAL && key0 + KT - 1 > q0) || (key0 + KT > N)) {
      // key = key0 + 4 hi + off, off a constant per register: the key is past
      // the row (causal) or past N iff off > lim
      int lim = N - 1 - key0 - 4 * hi;
      if constexpr (CAUSAL) lim = min(lim, qrow - key0 - 4 * hi);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
          sc[kb][r] = off > lim ? -INFINITY : sc[kb][r];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmax3(mx, sc[kb][r], sc[kb][r + 1]);
    mx = max_halves(mx);
    m_ref = __builtin_fmaxf(m_ref, __builtin_ceilf(mx * ct));  // ct > 0; -inf stays -inf
    // every row sees key 0 in tile 0, so its reference is finite from there on
    if (t == 0) m_base = (m_ref == -INFINITY) ? 0.f : m_ref;
    float shift = (m_ref == -INFINITY) ? 0.f : m_ref - m_base;
    const float moff = ((m_ref == -INFINITY) ? 0.f : m_ref) - pbias;
    float ls[4] = {-0.f, -0.f, -0.f, -0.f};  // x + -0 = x: the first adds fold away
#pragma unroll
    for (int w = 0; w < 8 * NSUB; ++w) {
      const int kb = w >> 2, r = 4 * (w & 3);
      const float e0 = exp2_fast(__builtin_fmaf(sc[kb][r], ct, -moff));  // P * 2^7 * mu
      const float e1 = exp2_fast(__builtin_fmaf(sc[kb][r + 1], ct, -moff));
      const float e2 = exp2_fast(__builtin_fmaf(sc[kb][r + 2], ct, -moff));
      const float e3 = exp2_fast(__builtin_fmaf(sc[kb][r + 3], ct, -moff));
      ls[w & 3] += (e0 + e1) + (e2 + e3);
      pb[w >> 3][w & 7] = (int)cvt_e4m3x4(e0, e1, e2, e3);
    }
    const float lsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
    // rare: scores grew by more than 2^64 over the first tile's; move the base
    // (an exact power of two) after every product that used the old one
    if (__any(shift > 64.f)) {
      const float f = exp2_fast(-shift);
      l_run *= f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= f;
      m_base += shift;
      shift = 0.f;
    }
    ishift = (int)shift;
    v_exp = vexp_t;
    l_run += lsum * __builtin_amdgcn_ldexpf(inv_f, ishift);
  };

  float ks_next, vs_next;  // block scales of the next stage's tile
  auto stage = [&](int t, const uint8_t* kt, const uint8_t* vt, uint8_t* k_fill, uint8_t* v_fill)
                   __attribute__((always_inline)) {
    // tile t's K and V block scales were read a stage earlier (drained by
    // its end-of-stage wait); read tile t + 1's now, ahead of the tile
    // requests, so no wait inside a part ever drains a tile request
    const float ksc = ks_next, vsc = vs_next;
    {
      const int sb = min(t + 1, nb - 1);  // one scale block per tile
      ks_next = ks[sb];
      vs_next = vs[sb];
    }
    if (grp == 0 && t >= 1) {  // stage 1 goes out with K_0 in the prologue
      if (t + 1 < T) issue_k(k_fill, t + 1);
      if (t < T) issue_v(v_fill, t);
    }
    mfma_part(t, kt, vt);
    __builtin_amdgcn_s_barrier();  // phase switch only (see the bf16 ping-pong kernel)
    vector_part(t, ksc, vsc);
    wait_vmem_all();
    __syncthreads();
  };

  // prologue: tile 0's scales, K_0, then stage 1 = {K_1, V_0^T}; wait for
  // Q, the scales and K_0 only
  ks_next = ks[0];
  vs_next = vs[0];
  if (grp == 0) {
    issue_k(Ks0, 0);
    issue_k(Ks1, 1);
    issue_v(Vs0, 0);
    static_assert(2 * IPL < 16, "the wait below encodes the requests of stage 1 in 4 bits");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * IPL));  // vmcnt(2 IPL); expcnt, lgkmcnt left open
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  }
  asm volatile("s_barrier" ::: "memory");
  if (grp == 1) __syncthreads();  // group 1 sits out slot 0
  stage(0, Ks0, Vs1, Ks1, Vs0);
  for (int t = 1; t <= T; t += 2) {
    stage(t, Ks1, Vs0, Ks0, Vs1);
    if (t + 1 <= T) stage(t + 1, Ks0, Vs1, Ks1, Vs0);
  }
  if (grp == 0) __syncthreads();  // group 0 sits out the last slot

  const float l_tot = sum_halves(l_run);
  if (qrow < N) {
    const float inv = 1.f / l_tot;
    float* orow = p.o + (size_t)bh * N * D + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 val = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                           o[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * g + 4 * hi) = val;
      }
    if (hi == 0) p.lse[(size_t)bh * N + qrow] = m_base * 0.6931471805599453f + __logf(l_tot);
  }
}

}  // namespace

hipError_t launch_fp8_prep(const Fp8PrepParams& p, int d, hipStream_t stream) {
  if (d != 128) return hipErrorInvalidValue;
  const int nb = (p.N + 127) / 128;
  const unsigned grid = (unsigned)nb * (unsigned)p.B * (unsigned)p.H;
  if (!p.per_tensor) {
    hipLaunchKernelGGL(fp8_prep_kernel<kPrepFused>, dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(fp8_prep_kernel<kPrepAmaxOnly>, dim3(grid), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(fp8_prep_kernel<kPrepGlobalScale>, dim3(grid), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(fp8_tensor_scale_kernel, dim3(1), dim3(1024), 0, stream, p.scale, (int)grid,
                     p.signs ? 11.313708498984761f : 1.f, p.pow2);
  return hipGetLastError();
}

bool fwd_fp8_pingpong(int N, bool causal) {
  // the ping-pong kernel for non-causal N >= 1024 and causal N >= 4096
  // (same-box measurements with 128-key tiles, 30-60 launches back to back:
  // 1.05-1.10 x the four-wave kernel non-causal from N = 1024; causal
  // against the one-buffer, three-workgroup four-wave kernel 0.93-0.95 x at
  // N = 1024-2048, 1.02 x at N = 4096, 1.06 x from N = 8192)
  return causal ? N >= 4096 : N >= 1024;
}

int fwd_fp8_ref_block(int N, bool causal) { return fwd_fp8_pingpong(N, causal) ? kPPKeys : kBC; }

hipError_t launch_fwd_fp8(const FwdFp8Params& p, int d, bool causal, hipStream_t stream) {
  if (d != 128) return hipErrorInvalidValue;
  if (fwd_fp8_pingpong(p.N, causal)) {
    const int nq = (p.N + 255) / 256;
    const unsigned grid = (unsigned)nq * (unsigned)p.B * (unsigned)p.H;
    if (causal)
      hipLaunchKernelGGL(fwd_fp8_pp_kernel<true>, dim3(grid), dim3(512), 0, stream, p);
    else
      hipLaunchKernelGGL(fwd_fp8_pp_kernel<false>, dim3(grid), dim3(512), 0, stream, p);
    return hipGetLastError();
  }
  const int nq = (p.N + kBR - 1) / kBR;
  const unsigned grid = (unsigned)nq * (unsigned)p.B * (unsigned)p.H;
  if (causal)
    hipLaunchKernelGGL(fwd_fp8_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(fwd_fp8_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa
