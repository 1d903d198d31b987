// Fused exact attention forward, bf16 operands, for gfx950 (MI355X).
//
// What is computed: O = softmax(scale * Q K^T) V and lse per query row, with
// the online-softmax recurrence over key tiles (running max m, running sum
// l, rescaled accumulator; wmrh.cn FlashAttention V3 article, section 二.1;
// FA3 explainer "FlashAttention-3：用异步流水榨出 Hopper 的 Attention 性能",
// section "Online Softmax 仍是精确合并的核心").  The N x N score matrix only
// ever exists as one 32 x 32 register tile per matrix instruction.
//
// Work decomposition (FA3 explainer, section "FA2 到 H100 后，瓶颈为什么又变了":
// parallelism over batch, heads and query tiles): one workgroup of 4 waves
// per (batch, head, 128-row query tile); each wave owns 32 query rows.
//
// Per wave the products are computed transposed, S^T = K Q^T and
// O^T = V^T P^T, so that a lane owns ONE query row (column L & 31 of every
// accumulator) and 16 of the 32 keys of each 32-key block.  The row max is
// then 31 in-lane max operations plus one exchange with the other half
// wave, the row sum needs no exchange until the epilogue, and the S^T
// accumulator registers are, after the exp and the bf16 cast, exactly the
// B operand of the PV product (the key permutation they carry is matched by
// the layout of V in LDS, the same trick the FA3 explainer's section
// "FP8 路径的第一个问题：WGMMA Layout" describes for P and V).
//
// Data path per key tile j (FA3 explainer, sections "第一层重叠" and
// "Circular Buffer 为什么不能无限加深"): K_j and V_j are read from HBM once
// per workgroup into a 2-stage LDS ring (stage = j mod 2) while tile j-1 is
// being consumed (the next tile's global loads are issued before the PV
// products of the current one); Q stays in VGPRs for the whole loop.  K is stored
// row-major with an XOR swizzle of 16-byte chunks (conflict-free A-operand
// reads), V is stored as [key/4][d][key%4] so that the transposed operand
// V^T is read with two 8-byte loads per matrix instruction.
//
// Causal (FA3 explainer, section "为什么 Causal Shape 可能更难调度"): a
// workgroup only visits key tiles up to its last query row, only tiles that
// cross a wave's diagonal are masked element-wise, waves whose rows all lie
// above a tile skip it, and the heaviest query tiles are launched first.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kQW = 32;              // query rows per wave
constexpr int kBR = kWaves * kQW;    // query rows per workgroup
constexpr int kThreads = kWaves * 64;

template <int D> struct Bf16Cfg;
template <> struct Bf16Cfg<64> { static constexpr int BC = 64; static constexpr int MINB = 2; };
template <> struct Bf16Cfg<128> { static constexpr int BC = 64; static constexpr int MINB = 2; };
template <> struct Bf16Cfg<256> { static constexpr int BC = 32; static constexpr int MINB = 1; };

// XOR applied to the 16-byte chunk index of K row r in LDS: makes the 16
// rows read together by a ds_read_b128 land on 16 distinct bank groups.
template <int D> __device__ __forceinline__ int k_swizzle(int r) {
  if constexpr (D == 64) return (r >> 1) & 7;  // 128-byte rows: two rows per 256 bytes
  else return r & 15;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, Bf16Cfg<D>::MINB) void fwd_bf16_kernel(FwdBf16Params p) {
  constexpr int BC = Bf16Cfg<D>::BC;
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int KCH = BC * CPR;        // chunks of a K tile
  constexpr int KPT = KCH / kThreads;  // K chunks per thread
  constexpr int VUN = (BC / 4) * CPR;  // (key quad, d chunk) units of a V tile
  constexpr int VPT = (VUN + kThreads - 1) / kThreads;  // V units per thread (the last may be partial)
  constexpr int NKB = BC / 32;         // 32-key blocks of S^T per tile
  constexpr int NDB = D / 32;          // 32-row blocks of O^T
  constexpr int NQS = D / 16;          // k-steps of S^T = K Q^T
  constexpr int NPS = BC / 16;         // k-steps of O^T = V^T P^T
  static_assert(KCH % kThreads == 0 && (VUN % kThreads == 0 || VUN < kThreads), "tile must split over the workgroup");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BC * D];

  const int N = p.N;
  const int BH = p.B * p.H;
  const int nq = (N + kBR - 1) / kBR;
  int bh, qt;
  if constexpr (CAUSAL) {
    // heaviest query tiles first; heads vary fastest so every XCD gets a mix
    qt = nq - 1 - (int)blockIdx.x / BH;
    bh = (int)blockIdx.x % BH;
  } else {
    const int w = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
    bh = w / nq;
    qt = w % nq;
  }

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const size_t base = (size_t)bh * N * D;
  const uint16_t* __restrict__ Qg = p.q + base;
  const uint16_t* __restrict__ Kg = p.k + base;
  const uint16_t* __restrict__ Vg = p.v + base;
  const int q0 = qt * kBR + wave * kQW;  // first query row of this wave
  const int qrow = q0 + l32;             // the query row this lane owns

  // Q^T as the B operand, resident for the whole loop: k-step s holds
  // d = 16 s + 8 hi .. +7 of row qrow.
  bf16x8 qreg[NQS];
  {
    const bool ok = qrow < N;
    const u32x4* src = reinterpret_cast<const u32x4*>(Qg + (size_t)(ok ? qrow : 0) * D);
#pragma unroll
    for (int s = 0; s < NQS; ++s) {
      u32x4 t = ok ? src[2 * s + hi] : u32x4{0, 0, 0, 0};
      qreg[s] = __builtin_bit_cast(bf16x8, t);
    }
  }

  const int kend = CAUSAL ? min(N, qt * kBR + kBR) : N;
  const int ntiles = (kend + BC - 1) / BC;

  u32x4 kpre[KPT];
  u32x4 vpre[VPT][4];

  auto load_tile = [&](int j) {
    const int key0 = j * BC;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int ci = tid + kThreads * i, row = ci / CPR, ch = ci % CPR, key = key0 + row;
      kpre[i] = key < N ? *reinterpret_cast<const u32x4*>(Kg + (size_t)key * D + ch * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int u = tid + kThreads * i, quad = u / CPR, ch = u % CPR;
      if (u >= VUN) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + 4 * quad + r;
        vpre[i][r] = key < N ? *reinterpret_cast<const u32x4*>(Vg + (size_t)key * D + ch * 8) : u32x4{0, 0, 0, 0};
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int ci = tid + kThreads * i, row = ci / CPR, ch = ci % CPR;
      *reinterpret_cast<u32x4*>(&Ks[buf][row * D + ((ch ^ k_swizzle<D>(row)) * 8)]) = kpre[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int u = tid + kThreads * i, quad = u / CPR, ch = u % CPR;
      if (u >= VUN) break;
      // 4 keys x 8 d  ->  8 d x 4 keys; dword m of a key row holds d = 2m, 2m+1
      u32x4* dst = reinterpret_cast<u32x4*>(&Vs[buf][(quad * D + ch * 8) * 4]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        u32x4 w;
        w[0] = perm_b32(vpre[i][1][m], vpre[i][0][m], 0x05040100u);
        w[1] = perm_b32(vpre[i][3][m], vpre[i][2][m], 0x05040100u);
        w[2] = perm_b32(vpre[i][1][m], vpre[i][0][m], 0x07060302u);
        w[3] = perm_b32(vpre[i][3][m], vpre[i][2][m], 0x07060302u);
        dst[m] = w;
      }
    }
  };

  float m_run = -INFINITY;  // running max of the raw scores of row qrow
  float l_run = 0.f;        // this half-wave's share of the running sum
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};

  const float c = p.c;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const bool more = j + 1 < ntiles;
    const int key0 = j * BC;
    const bool active = !CAUSAL || key0 <= q0 + kQW - 1;
    if (!active && more) load_tile(j + 1);
    if (active) {
      // ---- S^T = K_j Q^T ------------------------------------------------
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
        const int row = kb * 32 + l32;
        const uint16_t* krow = &Ks[buf][row * D];
        const int sw = k_swizzle<D>(row);
#pragma unroll
        for (int st = 0; st < NQS; ++st) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + (((2 * st + hi) ^ sw) * 8));
          s[kb] = mfma_bf16_32x32x16(a, qreg[st], s[kb]);
        }
      }
      // ---- mask (only tiles crossing the diagonal or the end of N) ------
      const bool need_mask = (CAUSAL && key0 + BC - 1 > q0) || (key0 + BC > N);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool dead = (CAUSAL && key > qrow) || key >= N;
            s[kb][r] = dead ? -INFINITY : s[kb][r];
          }
      }
      // ---- online softmax in the exp2 domain ------------------------------
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = fmax3(mx, s[kb][r], s[kb][r + 1]);
      mx = __builtin_fmaxf(mx, swap_halves(mx));
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float mc = m_use * c;
      const float alpha = exp2_fast(m_run * c - mc);
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = exp2_fast(__builtin_fmaf(s[kb][r], c, -mc));
          s[kb][r] = e;
          lsum += e;
        }
      l_run = alpha * l_run + lsum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      // P^T as bf16 B operands: k-step ks uses registers 8t..8t+7 of block ks/2
      bf16x8 pb[NPS];
#pragma unroll
      for (int ks = 0; ks < NPS; ++ks) {
        const int kb = ks >> 1, r0 = (ks & 1) * 8;
        u32x4 t;
        t[0] = pack_bf16x2(s[kb][r0 + 0], s[kb][r0 + 1]);
        t[1] = pack_bf16x2(s[kb][r0 + 2], s[kb][r0 + 3]);
        t[2] = pack_bf16x2(s[kb][r0 + 4], s[kb][r0 + 5]);
        t[3] = pack_bf16x2(s[kb][r0 + 6], s[kb][r0 + 7]);
        pb[ks] = __builtin_bit_cast(bf16x8, t);
      }
      // next tile's global loads fly while the PV products run
      if (more) load_tile(j + 1);
      // ---- O^T += V_j^T P^T -----------------------------------------------
      // k-step ks covers keys 16ks + 4hi + 0..3 and 16ks + 8 + 4hi + 0..3,
      // i.e. key quads 4ks + hi and 4ks + 2 + hi.
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int dcol = db * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < NPS; ++ks) {
          const u32x2 a0 = *reinterpret_cast<const u32x2*>(&Vs[buf][((4 * ks + hi) * D + dcol) * 4]);
          const u32x2 a1 = *reinterpret_cast<const u32x2*>(&Vs[buf][((4 * ks + 2 + hi) * D + dcol) * 4]);
          const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
          o[db] = mfma_bf16_32x32x16(__builtin_bit_cast(bf16x8, a), pb[ks], o[db]);
        }
      }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O / l, lse = m * scale + ln l ----------------------------
  const float l_tot = l_run + swap_halves(l_run);
  if (qrow < N) {
    const float inv = 1.f / l_tot;
    float* orow = p.o + base + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 val = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                           o[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * g + 4 * hi) = val;
      }
    if (hi == 0) p.lse[(size_t)bh * N + qrow] = m_run * p.scale + __logf(l_tot);
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdBf16Params& p, hipStream_t stream) {
  const int nq = (p.N + kBR - 1) / kBR;
  const unsigned grid = (unsigned)nq * (unsigned)p.B * (unsigned)p.H;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdBf16Params& p, int d, bool causal, hipStream_t stream) {
  switch (d) {
    case 64: return causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
    case 128: return causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
    case 256: return causal ? launch<256, true>(p, stream) : launch<256, false>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa
