// Fused exact attention forward, bf16 operands, for gfx950 (MI355X).
//
// What is computed: O = softmax(scale * Q K^T) V and lse per query row, with
// the online-softmax recurrence over key tiles (running max m, running sum
// l, rescaled accumulator; wmrh.cn FlashAttention V3 article, section 二.1;
// FA3 explainer "FlashAttention-3：用异步流水榨出 Hopper 的 Attention 性能",
// section "Online Softmax 仍是精确合并的核心").  The N x N score matrix only
// ever exists as 32 x 32 register tiles.
//
// Work decomposition (FA3 explainer, section "FA2 到 H100 后，瓶颈为什么又变了":
// parallelism over batch, heads and query tiles): one workgroup of NW waves
// per (batch, head, NW * 32 QB query rows); each wave owns QB blocks of 32
// query rows, so every K or V operand read from LDS feeds QB matrix
// instructions.  Every head size runs QB = 1: with QB = 2 a wave needs more
// than 256 registers and runs alone on its SIMD, which measured slower than
// two or three waves per SIMD with one block each.  The overlap of matrix
// and vector work is built into each wave's own instruction stream (below).
//
// Per wave the products are computed transposed, S^T = K Q^T and
// O^T = V^T P^T, so that a lane owns ONE query row (column L & 31 of every
// accumulator) and 16 of the 32 keys of each 32-key block.  The row max is
// then in-lane max operations plus one exchange with the other half wave,
// the row sum needs no exchange until the epilogue, and the S^T accumulator
// registers are, after exp2 and the bf16 cast, exactly the B operand of the
// PV product; the key permutation they carry is matched by how V^T is read
// (the FA3 explainer's section "FP8 路径的第一个问题：WGMMA Layout" describes
// the same trick of matching P's column order with V's row order).
//
// Data path (FA3 explainer, sections "第一层重叠：Producer 与 Consumer 并行",
// "Circular Buffer 为什么不能无限加深" and "第三层重叠：单个 Warpgroup 内跨迭代
// Pipeline"): K and V tiles go from HBM straight into LDS with buffer loads
// that write LDS directly (no register staging; rows past N read as zero
// through the buffer range check).  K runs one tile ahead of V: during the
// step for tile j the workgroup holds K_{j+1} and V_j, and the loads of
// K_{j+2} and V_{j+1} are in flight, in 2-slot rings (slot = tile mod 2).
// Inside a wave, S_{j+1} = K_{j+1} Q^T is issued on the matrix cores while
// the softmax of S_j runs on the vector ALUs (two S buffers, S_cur/S_next),
// and the row max of S_{j+1} is taken while O += V_j^T P_j^T runs.
// Q stays in VGPRs for the whole loop.  K is stored row-major with an XOR
// swizzle of 16-byte chunks (conflict-free A-operand reads); V is stored
// row-major with its own swizzle and read transposed with ds_read_b64_tr_b16.
//
// Softmax: exp2 domain (scale * log2 e folded into one FMA per score) and a
// lazy rescale: the running max used as the exponent reference only moves
// when some row of the wave has grown by more than 8 (log2 units); P is then
// at most 2^8 and O, l are rescaled only on those tiles.  O / l is exact
// whatever reference is used, so this changes no result beyond rounding.
//
// Causal (FA3 explainer, section "为什么 Causal Shape 可能更难调度"): a
// workgroup only visits key tiles up to its last query row, only tiles that
// cross a wave's diagonal are masked element-wise, waves whose rows all lie
// above a tile skip its products, and the heaviest query tiles launch first.
//
// d = 128 batches of 1024 or more query rows (512 non-causal, or causal in
// whole 256-row tiles) and non-causal d = 64 batches of 512 or more
// (fixed-length, or packed with such a longest sequence) run a second
// kernel, fwd_bf16_pp_kernel (below): eight waves per workgroup in two
// groups that take turns on each SIMD's matrix core (one group's products
// while the other group's softmax), the FA3 explainer's ping-pong
// scheduling mapped to wave pairs of a SIMD.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {
namespace {

// Per head size: QB 32-row query blocks per wave, NW waves per workgroup,
// BC keys per tile, MINB workgroups per CU.  Measured on MI355X: one query
// block per wave with two workgroups per CU (two waves per SIMD that
// interleave on the matrix cores) beats two blocks per wave at one wave per
// SIMD, which halves the LDS and L2 traffic per product but leaves a single
// wave unable to hide its own latencies.
//
// DMA_IN_BLOCK: where a wave issues its share of the next tiles' direct-to-LDS
// loads.  Issuing a step's loads back to back stalls the wave until the
// address unit has taken them; at d = 256 (one wave per SIMD, nothing to
// switch to) they go between the step's first products instead (same-box
// A/B: +3.5 % at N = 2048, +7-9 % at N = 16384).  At d = 64 and 128 the step
// keeps them ahead of its products: spread out they cost d = 64 spilled
// registers and short d = 128 sequences the unconditional requests past the
// last tile (-3 to -12 % at N <= 512).
template <int D> struct Bf16Cfg;
// ACC_IN_AGPR: the wave holds more than 256 registers, so the O accumulators
// live in AGPRs (the matrix instructions read and write them there).
template <> struct Bf16Cfg<64> {
  static constexpr int QB = 1, NW = 4, BC = 64, MINB = 3;
  static constexpr bool DMA_IN_BLOCK = false, ACC_IN_AGPR = false;
};
template <> struct Bf16Cfg<128> {
  static constexpr int QB = 1, NW = 4, BC = 64, MINB = 2;
  static constexpr bool DMA_IN_BLOCK = false, ACC_IN_AGPR = false;
};
template <> struct Bf16Cfg<256> {
  static constexpr int QB = 1, NW = 4, BC = 32, MINB = 1;
  static constexpr bool DMA_IN_BLOCK = true, ACC_IN_AGPR = true;
};
template <int D> constexpr int rows_per_workgroup() { return Bf16Cfg<D>::NW * 32 * Bf16Cfg<D>::QB; }
// Workgroups per CU the register budget is cut for.  At d = 64 a wave issues
// about as much vector work (exps, casts, sums) as matrix work per tile, so a
// third wave per SIMD hides the latency two leave open; the packed-batch
// variant keeps two (its extra sequence bookkeeping does not fit 168 VGPRs).
template <int D, bool VARLEN> constexpr int min_blocks() {
  return VARLEN && Bf16Cfg<D>::MINB > 2 ? 2 : Bf16Cfg<D>::MINB;
}

typedef __attribute__((address_space(3))) void* lds_void_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_t;

// XOR applied to the 16-byte chunk index of K row r: the rows read by one
// ds_read_b128 spread evenly over the LDS banks.
template <int D> __device__ __forceinline__ int k_swizzle(int r) {
  if constexpr (D == 64) return (r >> 1) & 7;  // 128-byte rows: two rows per 256 bytes
  else return r & 15;
}
// XOR for V rows, matched to the transposed read (8 rows x 4 chunks per
// instruction land on 16 distinct bank groups, twice each).
template <int D> __device__ __forceinline__ int v_swizzle(int r) {
  if constexpr (D == 64) return ((r >> 1) & 1) << 2;
  else return (r & 3) << 2;
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16 bytes per lane from buffer offset voff straight into LDS at dst + 16 * lane
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint16_t* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t)dst, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// four 16-bit elements through the transposing LDS read
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* src) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t)src);
}

// Instruction-group order for one pipeline step (compiler scheduling hints;
// masks: 0x008 matrix, 0x100 LDS read, 0x002 vector ALU).  QK phase: each
// K operand read feeds QB products and runs kKLead reads ahead, with kVPM
// softmax vector instructions between products; PV phase: each pair of
// transposed V reads feeds QB products, the V reads kVLead ahead, with kVPP
// row-max instructions of the next tile in between.  Values from a measured
// sweep on MI355X (all within +-3 %; no hints at all loses 5 % causal).
constexpr int kKLead = 2, kVLead = 4, kVPM = 3, kVPP = 2;
// NDMA direct-to-LDS loads (when the step issues them in its block) go one
// after each of the first NDMA K operand reads.
template <int NKR, int NVR, int QB, int NDMA>
__device__ __forceinline__ void schedule_step() {
  {
    __builtin_amdgcn_sched_group_barrier(0x100, kKLead, 0);
#pragma unroll
    for (int i = 0; i < NKR; ++i) {
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kVPM, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (i < NDMA) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kVLead, 0);
#pragma unroll
    for (int i = 0; i < NVR; ++i) {
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kVPP, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  }
}

// Where one (sequence, head) lives.  Fixed-length batch: [B, H, N, d] and
// [B, Hkv, Nk, d], rows d apart.  Packed batch: sequence bb's rows of the
// token-major tensors, H d (q, o) and Hkv d (k, v) apart, bounds clamped into
// the tensors.
template <bool VARLEN> struct SeqExtent {
  int N, Nk;              // query and key rows
  size_t qbase, kvbase;   // element offsets of row 0 of this (sequence, head)
  int qstride, kvstride;  // elements between consecutive rows
  size_t lbase;           // lse index of row 0
};
template <int D, bool VARLEN>
__device__ __forceinline__ SeqExtent<VARLEN> seq_extent(const FwdBf16Params& p, int bb, int hh, int hk) {
  SeqExtent<VARLEN> e;
  if constexpr (VARLEN) {
    const int q0s = min(max(p.cu_q[bb], 0), p.total_q), q1s = min(max(p.cu_q[bb + 1], q0s), p.total_q);
    const int k0s = min(max(p.cu_k[bb], 0), p.total_k), k1s = min(max(p.cu_k[bb + 1], k0s), p.total_k);
    e.N = q1s - q0s;
    e.Nk = k1s - k0s;
    e.qstride = p.H * D;
    e.kvstride = p.Hkv * D;
    e.qbase = (size_t)q0s * e.qstride + (size_t)hh * D;
    e.kvbase = (size_t)k0s * e.kvstride + (size_t)hk * D;
    e.lbase = (size_t)hh * p.total_q + q0s;
  } else {
    e.N = p.N;
    e.Nk = p.Nk;
    e.qstride = D;
    e.kvstride = D;
    e.qbase = ((size_t)bb * p.H + hh) * e.N * D;
    e.kvbase = ((size_t)bb * p.Hkv + hk) * e.Nk * D;
    e.lbase = ((size_t)bb * p.H + hh) * e.N;
  }
  return e;
}

template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(Bf16Cfg<D>::NW * 64, (min_blocks<D, VARLEN>())) void fwd_bf16_kernel(FwdBf16Params p) {
  using Cfg = Bf16Cfg<D>;
  constexpr int QB = Cfg::QB, NW = Cfg::NW, BC = Cfg::BC;
  constexpr int QW = 32 * QB;                 // query rows per wave
  constexpr int BR = NW * QW;                 // query rows per workgroup
  constexpr int ROWB = D * 2;                 // bytes per K/V row
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int INSTR = BC * ROWB / 1024;     // 1 KB wave-loads per tile
  constexpr int IPW = INSTR / NW;             // ... per wave
  constexpr int RPI = 1024 / ROWB;            // rows per wave-load
  constexpr int NKB = BC / 32;                // 32-key blocks of S^T per tile
  constexpr int NDB = D / 32;                 // 32-row blocks of O^T
  constexpr int NQS = D / 16;                 // k-steps of S^T = K Q^T
  constexpr int NPS = BC / 16;                // k-steps of O^T = V^T P^T
  static_assert(INSTR % NW == 0, "tile must split over the waves");
  static_assert(BC % 32 == 0, "key tiles are whole 32-key blocks of S^T");

  // one LDS object per ring slot, addressed with compile-time slot numbers,
  // so the compiler can tell the slot being filled from the slots being read
  __shared__ __attribute__((aligned(1024))) uint16_t Ks0[BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Ks1[BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Vs0[BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t Vs1[BC * D];

  const int BH = p.B * p.H;
  const int nq = (p.N + BR - 1) / BR;  // query tiles (of the longest sequence when VARLEN)
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
  // KV head of this query head: each KV head serves H / Hkv consecutive query heads
  const int bb = bh / p.H, hh = bh - bb * p.H;
  const int hk = hh / (p.H / p.Hkv);

  const SeqExtent<VARLEN> ex = seq_extent<D, VARLEN>(p, bb, hh, hk);
  const int N = ex.N, Nk = ex.Nk, qstride = ex.qstride, kvstride = ex.kvstride;
  const size_t qbase = ex.qbase, kvbase = ex.kvbase, lbase = ex.lbase;
  if (VARLEN && qt * BR >= N) return;  // past this sequence's queries: the whole workgroup leaves
  const int off = Nk - N;  // causal alignment: query i sees keys j <= i + off

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int q0 = qt * BR + wave * QW;  // first query row of this wave
  int qrow[QB];                        // the query rows this lane owns
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) qrow[qb] = q0 + 32 * qb + l32;

  // Q^T as B operands, resident for the whole loop: block qb, k-step s holds
  // d = 16 s + 8 hi .. +7 of row qrow[qb].
  bf16x8 qreg[QB][NQS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const bool ok = qrow[qb] < N;
    const u32x4* src = reinterpret_cast<const u32x4*>(p.q + qbase + (size_t)(ok ? qrow[qb] : 0) * qstride);
#pragma unroll
    for (int s = 0; s < NQS; ++s) {
      const u32x4 t = ok ? src[2 * s + hi] : u32x4{0, 0, 0, 0};
      qreg[qb][s] = __builtin_bit_cast(bf16x8, t);
    }
  }

  const int kend = CAUSAL ? min(Nk, qt * BR + BR + off) : Nk;
  const int ntiles = kend > 0 ? (kend + BC - 1) / BC : 0;

  // ---- direct-to-LDS tile loads -------------------------------------------
  // Wave-load i of wave w fills LDS bytes [(IPW w + i) KB, +1 KB) of the
  // slot: RPI rows; lane L writes physical chunk L % CPR of row L / CPR and
  // therefore fetches the logical chunk that the swizzle puts there.
  // The buffer range ends with this head's last key row, so rows past Nk
  // (also the next sequence's rows in a packed batch) read as zero.
  const int kvrowb = kvstride * 2;  // bytes between K/V rows in memory
  const int kvbytes = Nk > 0 ? (Nk - 1) * kvrowb + ROWB : 0;
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(p.k + kvbase, kvbytes);
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(p.v + kvbase, kvbytes);
  int koff[IPW], voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int row = (wave * IPW + i) * RPI + lane / CPR, pc = lane % CPR;
    koff[i] = row * kvrowb + ((pc ^ k_swizzle<D>(row)) * 16);
    voff[i] = row * kvrowb + ((pc ^ v_swizzle<D>(row)) * 16);
  }
  auto issue = [&](const __amdgpu_buffer_rsrc_t& r, uint16_t* dst, const int (&off)[IPW], int j) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) lds_dma16(r, dst + (wave * IPW + i) * 512, off[i] + j * BC * kvrowb);
  };

  // S^T = K Q^T: each K operand (row kb*32 + l32, chunk 2 st + hi) feeds QB products
  auto qk = [&](f32x16 (&s)[QB][NKB], const uint16_t* ks) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
    for (int st = 0; st < NQS; ++st)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int row = kb * 32 + l32;
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&ks[row * D + (((2 * st + hi) ^ k_swizzle<D>(row)) * 8)]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma_bf16_32x32x16(a, qreg[qb][st], s[qb][kb]);
      }
  };

  // V^T A-operand via the transposed read: within each 16-lane group, source
  // lane s addresses row kbase + s/4, columns dbase + 4 (s%4) .. +3; lane i of
  // the group then receives column dbase + i, rows kbase .. kbase + 3.
  const int grp = lane >> 4, sl = lane & 15;
  const int v_row_in = sl >> 2;                        // + kbase
  const int v_col_in = 16 * (grp & 1) + 4 * (sl & 3);  // + 32 db
  auto read_vt = [&](const uint16_t* vs, int kbase, int db) __attribute__((always_inline)) -> i16x4 {
    const int row = kbase + v_row_in;
    const int col = 32 * db + v_col_in;
    const int e = row * D + (((col >> 3) ^ v_swizzle<D>(row)) << 3) + (col & 7);
    return lds_read_tr16(&vs[e]);
  };

  // row max of one S^T block set: in-lane, then with the other half wave
  auto rowmax = [&](const f32x16 (&s)[NKB]) -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmax3(mx, s[kb][r], s[kb][r + 1]);
    return max_halves(mx);
  };

  float m_run[QB], l_run[QB];  // exponent reference (raw score units), this half-wave's row sum
  f32x16 o[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[qb][db] = f32x16{};
  }
  const float c = p.c;
  const float lazy = kLazyLog2 / c;  // the rescale threshold in raw score units

  // one step for tile j: softmax of S_j (s_in, whose unmasked row max is in
  // mx), S_{j+1} into s_out (its row max left in mx), O += V_j^T P_j^T.  The
  // ring slots are passed as compile-time LDS objects:
  //   k_this: holds K_j until this step, then receives K_{j+2};  k_next: K_{j+1}
  //   v_this: V_j;  v_next: receives V_{j+1}
  auto step = [&](int j, f32x16 (&s_in)[QB][NKB], f32x16 (&s_out)[QB][NKB], float (&mx)[QB], uint16_t* k_this,
                  const uint16_t* k_next, const uint16_t* v_this, uint16_t* v_next) {
    wait_vmem_all();
    __syncthreads();  // V_j and K_{j+1} are in LDS; every wave is done with K_j and V_{j-1}
    const int key0 = j * BC;
    const bool skip = CAUSAL && key0 > q0 + QW - 1 + off;  // every row of this wave lies above tile j (and later ones)
    if (!Cfg::DMA_IN_BLOCK || skip) {
      if (j + 2 < ntiles) issue(rk, k_this, koff, j + 2);
      if (j + 1 < ntiles) issue(rv, v_next, voff, j + 1);
    }
    if (skip) return;

    // ---- mask (only tiles crossing the diagonal or the end of N) ----------
    const bool need_mask = (CAUSAL && key0 + BC - 1 > q0 + off) || (key0 + BC > Nk);
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool dead = (CAUSAL && key > qrow[qb] + off) || key >= Nk;
            s_in[qb][kb][r] = dead ? -INFINITY : s_in[qb][kb][r];
          }
        mx[qb] = rowmax(s_in[qb]);
      }
    }
    // ---- lazy rescale ---------------------------------------------------------
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) grow |= mx[qb] > m_run[qb] + lazy;
    if (__any(grow)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_new = __builtin_fmaxf(m_run[qb], mx[qb]);
        // 0 on a row's first visible tile; a row that has seen no key yet
        // (m_new = -inf, l = 0, O = 0) must not take (-inf) - (-inf) = NaN
        const float alpha = m_new == -INFINITY ? 1.f : exp2_fast((m_run[qb] - m_new) * c);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          // With AGPR accumulators the operands of this (rare) multiply are
          // pinned to AGPRs on both sides (empty asm, "a" constraint): the
          // copy to vector registers and back then stays inside the branch.
          // Left to itself the compiler kept a vector-register copy of all
          // of O at the top of every step (128 AGPR reads per 32-key tile,
          // about half the vector work of a d = 256 step).
          if constexpr (Cfg::ACC_IN_AGPR) asm volatile("" : "+a"(o[qb][db]));
          o[qb][db] *= alpha;
          if constexpr (Cfg::ACC_IN_AGPR) asm volatile("" : "+a"(o[qb][db]));
        }
        m_run[qb] = m_new;
      }
    }

    // ---- one branch-free block: S_{j+1} = K_{j+1} Q^T on the matrix cores
    // while exp2 / bf16 cast / row sums of S_j run on the vector ALUs; then
    // O^T += V_j^T P_j^T while the row max of S_{j+1} is taken.  For the
    // last tile the first product reads a stale slot and is never used.
    if constexpr (Cfg::DMA_IN_BLOCK) {
      // this wave's share of K_{j+2} and V_{j+1}, spread between the products
      // below (past the last tile the range check reads zeros into a slot
      // that is not read again)
      issue(rk, k_this, koff, j + 2);
      issue(rv, v_next, voff, j + 1);
    }
    qk(s_out, k_next);
    bf16x8 pb[QB][NPS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mc = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb] * c;
      float ls[4] = {-0.f, -0.f, -0.f, -0.f};  // fp32 partial row sums (four short chains; x + -0 = x)
#pragma unroll
      for (int ks = 0; ks < NPS; ++ks) {
        const int kb = ks >> 1, r0 = (ks & 1) * 8;
        u32x4 t;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float e0 = exp2_fast(__builtin_fmaf(s_in[qb][kb][r0 + 2 * h], c, -mc));
          const float e1 = exp2_fast(__builtin_fmaf(s_in[qb][kb][r0 + 2 * h + 1], c, -mc));
          t[h] = pack_bf16x2(e0, e1);
          ls[h] += e0 + e1;
        }
        pb[qb][ks] = __builtin_bit_cast(bf16x8, t);
      }
      l_run[qb] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    }
    // k-step ks covers keys 16ks + 4hi + 0..3 (first read) and 16ks + 8 + 4hi
    // + 0..3 (second read): the key order of the P^T registers.
#pragma unroll
    for (int ks = 0; ks < NPS; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const i16x4 a0 = read_vt(v_this, 16 * ks + 4 * hi, db);
        const i16x4 a1 = read_vt(v_this, 16 * ks + 8 + 4 * hi, db);
        const u32x2 w0 = __builtin_bit_cast(u32x2, a0), w1 = __builtin_bit_cast(u32x2, a1);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma_bf16_32x32x16(a, pb[qb][ks], o[qb][db]);
      }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mx[qb] = rowmax(s_out[qb]);
    schedule_step<NKB * NQS, NPS * NDB, QB, Cfg::DMA_IN_BLOCK ? 2 * IPW : 0>();
  };

  // ---- prologue: K_0, V_0, K_1 in flight; S_0 and its row max ---------------
  f32x16 sa[QB][NKB], sb[QB][NKB];
  float mx[QB];
  if (ntiles > 0) {
    issue(rk, Ks0, koff, 0);
    issue(rv, Vs0, voff, 0);
  }
  if (ntiles > 1) issue(rk, Ks1, koff, 1);
  wait_vmem_all();
  __syncthreads();
  qk(sa, Ks0);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) mx[qb] = rowmax(sa[qb]);
  for (int j = 0; j < ntiles; j += 2) {
    step(j, sa, sb, mx, Ks0, Ks1, Vs0, Vs1);
    if (j + 1 < ntiles) step(j + 1, sb, sa, mx, Ks1, Ks0, Vs1, Vs0);
  }

  if constexpr (Cfg::DMA_IN_BLOCK) wait_vmem_all();  // the last (unused) requests land before the ring is reused
  // ---- epilogue: O / l, lse = m * scale + ln l ----------------------------
  // A lane holds 16-byte pieces of ONE output row, so storing straight from
  // the accumulators writes 32 bytes into each of 32 rows per instruction.
  // Where a wave's fp32 tile fits one ring slot (d = 64, 128), it goes
  // through LDS first (16-byte chunks XOR-swizzled by row: conflict-free on
  // both sides) and leaves as whole rows, 1 KB of consecutive bytes per
  // instruction.
  constexpr int CPO = D / 4;  // 16-byte chunks per fp32 output row
  constexpr bool kStageO = QB == 1 && 32 * D * 4 <= BC * D * 2;
  float inv[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = sum_halves(l_run[qb]);
    // a row that sees no key (only when N > Nk, causal) has l = 0: O = 0, lse = -inf
    inv[qb] = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow[qb] < N && hi == 0) p.lse[lbase + qrow[qb]] = m_run[qb] * p.scale + __logf(l_tot);
  }
  if constexpr (kStageO) {
    __syncthreads();  // every wave is done with the ring (no tile loads are in flight)
    float* st = reinterpret_cast<float*>(wave == 0 ? Ks0 : wave == 1 ? Ks1 : wave == 2 ? Vs0 : Vs1);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 8 * db + 2 * g + hi;  // chunk of d = 32 db + 8 g + 4 hi .. +3
        const f32x4 val = {o[0][db][4 * g] * inv[0], o[0][db][4 * g + 1] * inv[0], o[0][db][4 * g + 2] * inv[0],
                           o[0][db][4 * g + 3] * inv[0]};
        *reinterpret_cast<f32x4*>(st + l32 * D + ((c ^ (l32 & (CPO - 1))) * 4)) = val;
      }
    constexpr int RPS = 64 / CPO;  // rows per store instruction
#pragma unroll
    for (int t = 0; t < 32 / RPS; ++t) {
      const int r = t * RPS + lane / CPO, c = lane % CPO;
      const f32x4 val = *reinterpret_cast<const f32x4*>(st + r * D + ((c ^ (r & (CPO - 1))) * 4));
      if (q0 + r < N) *reinterpret_cast<f32x4*>(p.o + qbase + (size_t)(q0 + r) * qstride + 4 * c) = val;
    }
  } else {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (qrow[qb] < N) {
        float* orow = p.o + qbase + (size_t)qrow[qb] * qstride;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 val = {o[qb][db][4 * g] * inv[qb], o[qb][db][4 * g + 1] * inv[qb],
                               o[qb][db][4 * g + 2] * inv[qb], o[qb][db][4 * g + 3] * inv[qb]};
            *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * g + 4 * hi) = val;
          }
      }
    }
  }
}

// d = 128 (and non-causal d = 64) with an explicit ping-pong between two wave groups (FA3 explainer,
// section "第二层重叠：Ping-Pong Scheduling"): eight waves per workgroup,
// 32 query rows each; waves w and w + 4 share a SIMD.  The step of tile t is
// split into a matrix part (S_t = K_t Q^T and O += V_{t-1}^T P_{t-1}^T) and a
// vector part (mask, row max, rescale, exps and row sums of S_t).  In every
// slot one group runs its matrix part while the other runs its vector part,
// with a workgroup barrier between slots, so the two waves of a SIMD take
// turns on the matrix core instead of contending for it.
//   slot 2t:     group 0 matrix(t),  group 1 vector(t - 1)
//   slot 2t + 1: group 0 vector(t),  group 1 matrix(t)
// Stage t = {K_t, V_{t-1}} stays in LDS through slots 2t and 2t + 1, in a
// ring of four slots (128 KB at d = 128; after the loop each wave stages its
// output tile in one of the ring's eight tile buffers).  Each group issues
// half of a stage's direct-to-LDS loads inside its vector part (group 0 the
// K tile, group 1 the V tile): issuing a stage's 32 one-KB loads stalls the
// issuing waves for about 300 cycles (the address unit takes them one after
// another), which inside a matrix part idles the matrix core and inside one
// vector part lengthens the other group's slot; split over both vector parts
// it hides beside the other group's products.  With four slots every tile
// is requested three stages ahead and waited for at the end of a matrix
// part, where the vector part of the other group still runs.
template <int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(512, D == 64 ? 2 : 1) void fwd_bf16_pp_kernel(FwdBf16Params p) {
  constexpr int BC = D == 256 ? 32 : 64, NW = 8, QW = 32, BR = NW * QW;
  constexpr int ROWB = D * 2, CPR = D / 8;
  constexpr int INSTR = BC * ROWB / 1024;  // 1 KB wave-loads per tile
  constexpr int IPW = INSTR / NW;
  constexpr int RPI = 1024 / ROWB;
  constexpr int NKB = BC / 32, NDB = D / 32, NQS = D / 16, NPS = BC / 16;

  // The ring is one LDS array: a slot's address is then a constant offset of
  // one base, which the reads' immediate offset field takes.  With one array
  // per slot the compiler kept a separate set of per-lane read addresses for
  // each slot (about 40 more VGPRs).  Slot i holds K in tile buffer i and V
  // in tile buffer 4 + i.
  __shared__ __attribute__((aligned(1024))) uint16_t ring[8 * BC * D];
  auto Ks = [&](int i) __attribute__((always_inline)) { return ring + i * BC * D; };
  auto Vs = [&](int i) __attribute__((always_inline)) { return ring + (4 + i) * BC * D; };
  // O is staged through LDS where a wave's fp32 tile fits a tile buffer (d = 64, 128)
  constexpr bool kStageO = QW * D * 4 <= BC * D * 2;

  const int BH = p.B * p.H;
  const int nq = (p.N + BR - 1) / BR;
  int bh, qt;
  if constexpr (CAUSAL) {
    causal_order(BH, nq, bh, qt);
  } else {
    const int w = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
    bh = w / nq;
    qt = w % nq;
  }
  const int bb = bh / p.H, hh = bh - bb * p.H;
  const int hk = hh / (p.H / p.Hkv);
  const SeqExtent<VARLEN> ex = seq_extent<D, VARLEN>(p, bb, hh, hk);
  const int N = ex.N, Nk = ex.Nk, qstride = ex.qstride;
  const size_t qbase = ex.qbase, kvbase = ex.kvbase, lbase = ex.lbase;
  if (VARLEN && qt * BR >= N) return;  // past this sequence's queries: the whole workgroup leaves
  const int off = Nk - N;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int grp = wave >> 2;
  // causal: group 0, which runs one slot ahead, takes the later 128 rows
  // (the ones with the most key tiles), so the workgroup ends with group 0's
  // last vector part rather than one slot after it
  const int q0 = qt * BR + (CAUSAL ? (wave ^ 4) : wave) * QW;
  const int qrow = q0 + l32;

  // Q^T operands through range-checked buffer loads (rows past N read as
  // zero): no branch around the loads, so the compiler can count them
  bf16x8 qreg[NQS];
  {
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(p.q + qbase, N > 0 ? ((N - 1) * qstride + D) * 2 : 0);
#pragma unroll
    for (int st = 0; st < NQS; ++st)
      qreg[st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, (qrow * qstride + (2 * st + hi) * 8) * 2, 0, 0));
    // keep them ahead of the tile requests: the counter drains in order
    __builtin_amdgcn_sched_barrier(0);
  }

  const int kend = CAUSAL ? min(Nk, qt * BR + BR + off) : Nk;
  const int T = kend > 0 ? (kend + BC - 1) / BC : 0;  // tiles of the workgroup
  const int lastkey = q0 + QW - 1 + off;             // this wave's last visible key (causal)
  const int Tw = CAUSAL ? (lastkey < 0 ? 0 : min(T, lastkey / BC + 1)) : T;  // tiles this wave uses

  // tile requests: the four waves of a group each load a quarter of a K tile
  // (group 0) or a V tile (group 1), 4 KB per wave and tile
  const int kvrowb = ex.kvstride * 2;
  const int kvbytes = Nk > 0 ? (Nk - 1) * kvrowb + ROWB : 0;
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(p.k + kvbase, kvbytes);
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(p.v + kvbase, kvbytes);
  constexpr int IPL = INSTR / 4;  // wave-loads per loading wave and tile
  const int lw = wave & 3;
  int koff[IPL], voff[IPL];
#pragma unroll
  for (int i = 0; i < IPL; ++i) {
    const int row = (lw * IPL + i) * RPI + lane / CPR, pc = lane % CPR;
    koff[i] = row * kvrowb + ((pc ^ k_swizzle<D>(row)) * 16);
    voff[i] = row * kvrowb + ((pc ^ v_swizzle<D>(row)) * 16);
  }
  auto issue = [&](const __amdgpu_buffer_rsrc_t& r, uint16_t* dst, const int (&of)[IPL], int j) {
#pragma unroll
    for (int i = 0; i < IPL; ++i) lds_dma16(r, dst + (lw * IPL + i) * 512, of[i] + j * BC * kvrowb);
  };

  const int grpv = lane >> 4, sl = lane & 15;
  const int v_row_in = sl >> 2;
  const int v_col_in = 16 * (grpv & 1) + 4 * (sl & 3);
  auto read_vt = [&](const uint16_t* vs, int kbase, int db) __attribute__((always_inline)) -> i16x4 {
    const int row = kbase + v_row_in;
    const int col = 32 * db + v_col_in;
    const int e = row * D + (((col >> 3) ^ v_swizzle<D>(row)) << 3) + (col & 7);
    return lds_read_tr16(&vs[e]);
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  f32x16 sc[NKB];
  bf16x8 pb[NPS];
  const float c = p.c;
  const float lazy = kLazyLog2 / c;

  // matrix part of stage t: S_t = K_t Q^T, then O^T += V_{t-1}^T P_{t-1}^T
  auto qk_part = [&](const uint16_t* kt) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sc[kb] = f32x16{};
#pragma unroll
    for (int st = 0; st < NQS; ++st)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int row = kb * 32 + l32;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kt[row * D + (((2 * st + hi) ^ k_swizzle<D>(row)) * 8)]);
        sc[kb] = mfma_bf16_32x32x16(a, qreg[st], sc[kb]);
      }
  };
  auto pv_part = [&](const uint16_t* vt) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < NPS; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const i16x4 a0 = read_vt(vt, 16 * ks + 4 * hi, db);
        const i16x4 a1 = read_vt(vt, 16 * ks + 8 + 4 * hi, db);
        const u32x2 w0 = __builtin_bit_cast(u32x2, a0), w1 = __builtin_bit_cast(u32x2, a1);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
        o[db] = mfma_bf16_32x32x16(a, pb[ks], o[db]);
      }
  };
  // K operand reads KL ahead of their products, transposed V reads VL ahead
  // (two per product); at d = 256 shorter leads keep the wave within 256 VGPRs
  // (d = 128: 5 and 8 measured 1.00-1.04 x over 3 and 4, outputs equal)
  constexpr int KL = D == 256 ? 1 : 5, VL = D == 256 ? 2 : 8;
  auto sched_qk = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x100, KL, 0);
#pragma unroll
    for (int i = 0; i < NQS * NKB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < NQS * NKB - KL) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  auto sched_pv = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x100, VL, 0);
#pragma unroll
    for (int i = 0; i < NPS * NDB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < NPS * NDB - VL / 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };
  auto mfma_part = [&](int t, const uint16_t* kt, const uint16_t* vt) __attribute__((always_inline)) {
    if (t < Tw) {
      qk_part(kt);
      sched_qk();
    }
    if (t >= 1 && t <= Tw) {
      pv_part(vt);
      sched_pv();
    }
  };

  // vector part of stage t: mask, row max, rescale, P_t = exp2 and row sums of S_t
  auto vector_part = [&](int t) __attribute__((always_inline)) {
    if (t >= Tw) return;
    const int key0 = t * BC;
    const bool need_mask = (CAUSAL && key0 + BC - 1 > q0 + off) || (key0 + BC > Nk);
    if (need_mask) {
      // as in the four-wave kernel: dead iff the register's key offset k > lim
      int lim = Nk - 1 - key0 - 4 * hi;
      if constexpr (CAUSAL) lim = min(lim, qrow + off - key0 - 4 * hi);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int k = kb * 32 + 8 * (r >> 2) + (r & 3);
          sc[kb][r] = k > lim ? -INFINITY : sc[kb][r];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmax3(mx, sc[kb][r], sc[kb][r + 1]);
    mx = max_halves(mx);
    if (__any(mx > m_run + lazy)) {
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : exp2_fast((m_run - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
    float ls[4] = {-0.f, -0.f, -0.f, -0.f};  // x + -0 = x: the first adds fold away
#pragma unroll
    for (int ks = 0; ks < NPS; ++ks) {
      const int kb = ks >> 1, r0 = (ks & 1) * 8;
      u32x4 w;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float e0 = exp2_fast(__builtin_fmaf(sc[kb][r0 + 2 * h], c, -mc));
        const float e1 = exp2_fast(__builtin_fmaf(sc[kb][r0 + 2 * h + 1], c, -mc));
        w[h] = pack_bf16x2(e0, e1);
        ls[h] += e0 + e1;
      }
      pb[ks] = __builtin_bit_cast(bf16x8, w);
    }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };

  // Both groups run the same sequence, group 1 one slot later: group 0's
  // matrix(t) falls in slot 2t and its vector(t) in 2t + 1, group 1's in
  // 2t + 1 and 2t + 2.  Stage s = {K_s, V_{s-1}} lives in ring slot s mod 4
  // and is read by the matrix parts of slots 2s and 2s + 1.  At the start of
  // its vector part of stage t, group 0 requests K_{t+3} and group 1 V_{t+2}
  // (both of stage t + 3, ring slot (t - 1) mod 4, whose last reader
  // finished in slot 2t - 1).  Each group waits for its requests at the end
  // of its matrix part of stage t + 2 (group 0 in slot 2t + 4, group 1 in
  // 2t + 5), before the barrier opening the slot after, so stage t + 3 is
  // complete before slot 2t + 6 first reads it.  Requests past the last tile
  // read zeros into a slot nobody reads again.
  auto stage = [&](int t, int slot) __attribute__((always_inline)) {
    mfma_part(t, Ks(slot), Vs(slot));
    __builtin_amdgcn_sched_barrier(0);         // every product issues before the phase switch
    __builtin_amdgcn_s_waitcnt(0x0F70 | IPL);  // vmcnt: all but this group's latest requests
    // phase switch: the tiles waited for above are next read two slots on;
    // the vector part touches no LDS and every K/V read of the matrix part is
    // consumed by its product before the wave gets here, so no fence
    __builtin_amdgcn_s_barrier();
    if (grp == 0) issue(rk, Ks((slot + 3) & 3), koff, t + 3);
    else issue(rv, Vs((slot + 3) & 3), voff, t + 2);
    vector_part(t);
    __syncthreads();
  };

  // prologue: group 0 requests K_0, K_1, K_2 and waits for K_0 (and Q),
  // group 1 requests V_0 and V_1 (past the keys the range check returns
  // zeros); the rest is waited for by the waits above, each in time
  if (grp == 0) {
    issue(rk, Ks(0), koff, 0);
    issue(rk, Ks(1), koff, 1);
    issue(rk, Ks(2), koff, 2);
    static_assert(2 * IPL <= 15, "the wait below encodes vmcnt in 4 bits");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * IPL));  // vmcnt(K_1's and K_2's requests)
  } else {
    issue(rv, Vs(1), voff, 0);
    issue(rv, Vs(2), voff, 1);
  }
  // K_0 landed (each loading wave waited for its share); later tiles may
  // still be in flight, so a plain barrier (the fence of __syncthreads would
  // drain them) that the compiler may not move LDS accesses across
  asm volatile("s_barrier" ::: "memory");
  if (grp == 1) __syncthreads();  // group 1 sits out slot 0
  for (int t = 0; t <= T; t += 4) {
    stage(t, 0);
    if (t + 1 <= T) stage(t + 1, 1);
    if (t + 2 <= T) stage(t + 2, 2);
    if (t + 3 <= T) stage(t + 3, 3);
  }
  if (grp == 0) __syncthreads();  // group 0 sits out the last slot
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the last (unused) requests land before the ring is reused
  __syncthreads();

  // epilogue: O / l, staged through LDS where it fits (wave w in tile buffer
  // w of the ring) and stored as whole rows; every wave is past its last ring
  // read (the final barrier above)
  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < N && hi == 0) p.lse[lbase + qrow] = m_run * p.scale + __logf(l_tot);
  if constexpr (kStageO) {
    constexpr int CPO = D / 4;  // 16-byte chunks per fp32 row
    float* st = reinterpret_cast<float*>(ring + wave * BC * D);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cc = 8 * db + 2 * g + hi;  // chunk of d = 32 db + 8 g + 4 hi .. +3
        const f32x4 val = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(st + l32 * D + ((cc ^ (l32 & (CPO - 1))) * 4)) = val;
      }
    constexpr int RPS = 64 / CPO;  // rows per store instruction
#pragma unroll
    for (int t = 0; t < 32 / RPS; ++t) {
      const int r = t * RPS + lane / CPO, cc = lane % CPO;
      const f32x4 val = *reinterpret_cast<const f32x4*>(st + r * D + ((cc ^ (r & (CPO - 1))) * 4));
      if (q0 + r < N) *reinterpret_cast<f32x4*>(p.o + qbase + (size_t)(q0 + r) * qstride + 4 * cc) = val;
    }
  } else if (qrow < N) {
    float* orow = p.o + qbase + (size_t)qrow * qstride;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 val = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * g + 4 * hi) = val;
      }
  }
}

// The ping-pong kernel takes d = 128 batches whose longest sequence has at
// least 1024 query rows, and from 512 rows non-causal ones and causal ones of
// whole 256-row tiles, fixed-length or packed; the others keep 128-row
// workgroups, which leave fewer idle rows and balance short causal grids
// better (same-box measurements with the four-slot ring: ping-pong 1.03-1.10 x
// from N = 1024 up, causal 1.03 x at N = 512 and 1.12 x at 768, but 0.94 x at
// N = 640, a half-empty last tile, and 0.90 x at N = 256; packed batches of
// 128-8192 rows 1.05-1.12 x).
// At d = 64 (127 VGPRs and a 64 KB ring: two workgroups per CU) it takes
// non-causal batches from 512 rows: 1.02 x at N = 512, 1.09-1.11 x from
// N = 1024, where causal ones stay on the three-workgroups-per-CU kernel
// (0.80-0.98 x there).  d = 256 needs more than 256 VGPRs (O 128, Q 64) and
// spills 12-13 in the loop (0.62-0.79 x).
inline bool use_pingpong(const FwdBf16Params& p, int d, bool causal) {
  if (d == 64) return !causal && p.N >= 512;
  return p.N >= 1024 || (p.N >= 512 && (!causal || p.N % 256 == 0));
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch(const FwdBf16Params& p, hipStream_t stream) {
  if constexpr (D == 128 || (D == 64 && !CAUSAL)) {
    if (use_pingpong(p, D, CAUSAL)) {
      const int nq = (p.N + 255) / 256;
      const unsigned grid = (unsigned)nq * (unsigned)p.B * (unsigned)p.H;
      if (grid == 0) return hipSuccess;
      hipLaunchKernelGGL((fwd_bf16_pp_kernel<D, CAUSAL, VARLEN>), dim3(grid), dim3(512), 0, stream, p);
      return hipGetLastError();
    }
  }
  constexpr int BR = rows_per_workgroup<D>();
  const int nq = (p.N + BR - 1) / BR;
  const unsigned grid = (unsigned)nq * (unsigned)p.B * (unsigned)p.H;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, VARLEN>), dim3(grid), dim3(Bf16Cfg<D>::NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <bool VARLEN>
hipError_t launch_any(const FwdBf16Params& p, int d, bool causal, hipStream_t stream) {
  switch (d) {
    case 64: return causal ? launch<64, true, VARLEN>(p, stream) : launch<64, false, VARLEN>(p, stream);
    case 128: return causal ? launch<128, true, VARLEN>(p, stream) : launch<128, false, VARLEN>(p, stream);
    case 256: return causal ? launch<256, true, VARLEN>(p, stream) : launch<256, false, VARLEN>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdBf16Params& p, int d, bool causal, hipStream_t stream) {
  return launch_any<false>(p, d, causal, stream);
}

hipError_t launch_fwd_bf16_varlen(const FwdBf16Params& p, int d, bool causal, hipStream_t stream) {
  return launch_any<true>(p, d, causal, stream);
}

}  // namespace fa
