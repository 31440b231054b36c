// Selected-block attention forward kernel for gfx950 (CDNA4).
//
// What it computes (vllm-omni PR #8335 "[Core] Add shared block-sparse
// attention adapters with FlashAttention-4", Purpose; diffusers
// examples/cosmos3/cosmos_parallel.py, cosmos3_cp_attention and
// build_gen_key_mask): for every query row of a query block, non-causal
// softmax attention over the keys of the KV blocks listed for that
// (batch, query head, query block), padded keys excluded, query head h
// reading KV head h / G in place. The dense case is the same kernel with the
// list "every non-empty block" generated in-kernel; the causal dense case
// (the understanding pathway's causal self-attention in cosmos3_cp_attention,
// bottom-right aligned as in mstar PR #927, automated review) cuts that list
// at the block's last reachable key and masks the diagonal stages.
//
// Structure: one workgroup per query block. Its rows form NQG = block_q / 32
// query groups and the keys are streamed in stages of 64, split into two key
// halves; wave (qh, kh) computes query rows [32 qh, 32 qh + 32) against keys
// [32 kh, 32 kh + 32) of every stage, so every K/V stage in LDS feeds all the
// block's rows. Each wave keeps its own partial softmax state; the two key
// halves are merged once at the end. At head_dim 128 a wave needs fewer than
// 256 registers, so every SIMD runs two waves (two 4-wave workgroups per CU
// at 64-row blocks, one 8-wave workgroup at 128-row blocks; a 256-row block
// runs as two 128-row workgroups on the same list); at head_dim 64 it needs
// fewer than 168 and a SIMD runs three (three 64-row workgroups per CU).
// While one wave waits (LDS, barrier, the HBM copies) another issues, and one
// wave's softmax overlaps another's matrix products.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the K fragment (A operand)
//    comes from LDS, Q^T (B operand) stays in registers for the whole
//    kernel. Each lane owns one query row and half of the 32 keys, so the
//    row max needs a single cross-lane step.
//  * Online softmax in fp32 in the log2 domain, the scale folded into one
//    FMA; the reference max of a row moves only when a stage max exceeds it
//    by more than 2^8 (lazy rescale), and the cross-lane step is skipped when
//    no lane comes near that. Row sums are accumulated on the vector ALU.
//  * O^T = V^T P^T with the same MFMA: P^T is the S^T accumulator converted
//    to bf16 in place (the contraction over keys is order-free, so the key
//    order of the accumulator layout is reused for V); V^T fragments come
//    from the row-major V tile through ds_read_b64_tr_b16.
//  * Inside a wave the QK^T MFMAs of the next stage are interleaved with the
//    exponentials of the current one, and the PV MFMAs with the row maxima
//    of the next.
//  * K and V stages move HBM -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging), XOR-swizzled in 16-byte chunks so that the K row reads and
//    the V transpose reads hit distinct banks, double buffered: K two stages
//    ahead, V one. One workgroup barrier per stage. Past the end of the list
//    the copies keep running on in-bounds rows, so they need no branch.
//  * Workgroups are renumbered so that each XCD works through a contiguous
//    range of (KV head, query block), keeping that range's K/V tiles in the
//    XCD's L2.

#include <type_traits>
#include <utility>

#include "internal.h"

namespace bsattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Chunk permutation of row `row` in an LDS tile with CPR 16-byte chunks.
// LDS serves 256 contiguous bytes per cycle. With 16 chunks per row (head
// dim 128) the permutation 4 (r % 4) + (r / 4) % 4 gives
//  * the K reads (16 lanes = 16 consecutive rows, one chunk each) 16
//    distinct chunk positions, and
//  * the V transpose reads (32 lanes = 4 consecutive rows x 4 adjacent
//    chunks) 16 distinct chunk positions.
// With 8 chunks per row two rows share a 256-byte line, and (r / 2) % 8
// keeps the K reads conflict-free. Both depend on r % 16 only.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CPR == 16) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    return (row >> 1) & (CPR - 1);
  }
}

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt
// left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  constexpr int imm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
  __builtin_amdgcn_s_waitcnt(imm);
}

// Workgroup barrier that orders LDS accesses only. Unlike __syncthreads()
// it does not wait for outstanding HBM->LDS copies, which stay in flight
// across it; their completion is awaited explicitly with wait_vmcnt.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// HBM->LDS copy of this wave's RPW rows (rows RPW w .. RPW w + RPW - 1) of a
// 64-row stage, with global_load_lds_dwordx4 in its scalar-base form: the LDS
// destination comes from M0 and the HBM address is a 64-bit scalar base plus
// a 32-bit per-lane offset, so a copy costs no vector ALU work. Instruction
// `it` moves 64 x 16 bytes = RPI whole rows. The lane's chunk within its row
// carries the XOR swizzle, which depends on the row modulo 16 only.
//
// The copies are issued from inline assembly, so the compiler does not track
// them: every read of a stage is preceded by an explicit wait_vmcnt and a
// workgroup barrier.
template <int D, int RPW>
struct StageCopy {
  static constexpr int CPR = D / 8;
  static constexpr int RPI = 64 / CPR;
  static constexpr int NL = RPW / RPI;  // instructions per wave and stage
  static_assert(NL * RPI == RPW && NL >= 1, "rows per wave");
  uint32_t voff[NL];                   // per-lane byte offsets

  // The swizzle follows the row's position in the stage (RPW wave + row).
  __device__ __forceinline__ void init(int64_t row_stride, int lane, int wave) {
#pragma unroll
    for (int it = 0; it < NL; ++it) {
      const int row = it * RPI + lane / CPR;
      const int lch = (lane % CPR) ^ swz<CPR>(wave * RPW + row);
      voff[it] = (uint32_t)((row * row_stride + lch * 8) * 2);
    }
  }
  template <int IT>
  __device__ __forceinline__ void one(const uint16_t* rows, uint32_t lds) const {
    asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff[IT]), "s"(rows), "s"(lds), "i"(IT * 1024)
                 : "memory", "m0");
  }
  // `rows`: uniform address of this wave's first row; `lds`: LDS byte address
  // of this wave's part of the stage. `it` is a constant after unrolling.
  __device__ __forceinline__ void issue_one(int it, const uint16_t* rows, uint32_t lds) const {
    switch (it) {
      case 0: one<0>(rows, lds); break;
      case 1: one<1 % NL>(rows, lds); break;
      case 2: one<2 % NL>(rows, lds); break;
      case 3: one<3 % NL>(rows, lds); break;
      default: break;
    }
  }
  __device__ __forceinline__ void issue(const uint16_t* rows, uint32_t lds) const {
#pragma unroll
    for (int it = 0; it < NL; ++it) issue_one(it, rows, lds);
  }
};

// Uniform 32-bit load through the scalar data cache (the index list is
// read-only here); waits for its own completion.
__device__ __forceinline__ int scalar_load_i32(const int32_t* ptr) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
  return v;
}

// Lanes l and l ^ 32 hold the same query row (different keys).
__device__ __forceinline__ float max_with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D, int BK, int NQG, int MODE>
__device__ __forceinline__ void attn_fwd_body(const AttnParams& p, uint16_t* __restrict__ smem) {
  constexpr bool DENSE = MODE != kSparse;    // the list is every non-empty block
  constexpr bool CAUSAL = MODE == kCausal;   // ... cut to the causal range
  constexpr int CPR = D / 8;
  constexpr int KS = D / 16;     // MFMA k-steps over D (QK^T MFMAs per stage)
  constexpr int DT = D / 32;     // output 32-row tiles over D
  constexpr int SPB = BK / 64;   // 64-key stages per block
  constexpr int STAGE = 64 * D;  // elements of one K or V stage
  static_assert(SPB == 1 || SPB == 2, "block_k 64 or 128");
  constexpr int NW = 2 * NQG;    // waves: NQG query groups of 32 rows x 2 key halves
  constexpr int RPW = 64 / NW;   // stage rows copied by each wave
  using Copy = StageCopy<D, RPW>;
  // A row moves its reference max only when a stage max exceeds it by more
  // than this many powers of two; until then probabilities are taken against
  // the stale max and stay below 2^8, far from fp32 or bf16 overflow.
  constexpr float kRescaleSlack = 8.0f;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qh = wave >> 1;  // 32-row query group
  const int kh = wave & 1;   // key half of every stage
  const int col = lane & 31;
  const int half = lane >> 5;

  // Workgroup w runs on XCD w % 8. The work is the (batch, KV head, query
  // block, head-in-group, part) order; a query block of more than 128 rows
  // is split into parts of 32 NQG rows, one workgroup each, reading the same
  // list. Each XCD takes a contiguous range of that order, so neighbours
  // (the heads of a group, adjacent query blocks: similar lists) share its
  // L2. When the K/V of all heads would not fit in the 256 MB last-level
  // cache together, the XCDs instead split every (batch, KV head) eight ways
  // and move through the KV heads in step, so only one head's K/V is live;
  // the grid is then padded to a multiple of eight per (batch, KV head).
  const int w = blockIdx.x;
  const int xcd = w & 7, kx = w >> 3;
  int lin, bg;
  if (p.head_sync) {
    const int tot = p.nq * p.group * p.qparts;  // workgroups per (batch, KV head)
    const int per = (tot + 7) >> 3;
    bg = kx / per;
    lin = xcd * per + kx % per;
    if (lin >= tot) return;  // padding: the whole workgroup leaves before any barrier
  } else {
    const int nwg = p.n_wg, per = nwg >> 3, rem = nwg & 7;
    const int all = xcd * per + min(xcd, rem) + kx;
    const int tot = p.nq * p.group * p.qparts;
    bg = all / tot;
    lin = all % tot;
  }
  const int part = lin % p.qparts;
  int t = lin / p.qparts;
  const int hig = t % p.group;
  const int i = t / p.group;
  const int g = bg % p.hkv;
  const int b = bg / p.hkv;
  const int h = g * p.group + hig;
  const int row0 = (i * p.qparts + part) * (32 * NQG);
  const int qrow = row0 + 32 * qh + col;


  int nblk;
  const int32_t* idx_row = nullptr;
  if constexpr (CAUSAL) {
    // Blocks whose first real key has a rank within reach of the block's last
    // real row (rank <= t + causal_off); their real keys are ranked in block
    // order: prefix block n from n BK, generation block m from
    // kv_prefix_valid + m BK.
    const int last_rank = min(row0 + 32 * NQG, p.q_valid) - 1 + p.causal_off;
    int n_pre = 0, n_gen = 0;
    if (last_rank >= 0) {
      n_pre = min(p.n_forced, last_rank / BK + 1);
      if (last_rank >= p.kv_prefix_valid)
        n_gen = min(p.n_cand, (last_rank - p.kv_prefix_valid) / BK + 1);
    }
    nblk = n_pre + n_gen;
  } else if constexpr (DENSE) {
    nblk = p.n_forced + p.n_cand;
  } else {
    const int64_t row_id = ((int64_t)b * p.hq + h) * p.nq + i;
    nblk = min(max(scalar_load_i32(p.cnt + row_id), 0), p.idx_row_stride);
    idx_row = p.idx + row_id * p.idx_row_stride;
  }
  if (row0 >= p.q_valid || p.nk == 0) nblk = 0;
  const int nst = nblk * SPB;  // stages
  // Where in its list this workgroup starts (it wraps around to the start).
  // With two workgroups per CU the dispatcher settles into rounds of 64 per
  // XCD whose second 32 start about half a workgroup lifetime after the
  // first 32 (measured). Starting those at the middle of their lists keeps
  // all the XCD's workgroups at about the same place in the KV sequence at
  // any time, so they share the blocks in L2. At head_dim 64 a CU holds
  // three 64-row workgroups, and the three cohorts of 32 start a third of
  // their lists apart. The order depends on blockIdx only, so results stay
  // bitwise reproducible.
  const int cohort = (w >> 8) % (D == 64 ? 3 : 2);  // (w / 8) / 32: cohorts of 32 per XCD
  const int n_first = (NQG == 2) ? (cohort * nblk) / (D == 64 ? 3 : 2) : 0;
  // The list, 64 positions at a time: lane l of lw_cur holds list position
  // 64 lw_c + l (after the rotation), lw_next the next 64. Each chunk is one
  // vector load issued a whole chunk before its first use, so reading the
  // list never waits on memory.
  int lw_cur = -1, lw_next = -1, lw_c = 0;
  auto load_chunk = [&](int c) -> int {
    const int pos = c * 64 + lane;
    int n = pos + n_first;
    if (n >= nblk) n -= nblk;
    return pos < nblk ? idx_row[n] : -1;
  };
  if constexpr (!DENSE) {
    lw_cur = load_chunk(0);
    lw_next = load_chunk(1);
  }
  // Q^T fragments (B operand): the lane holds q[qrow][16 ks + 8 half .. +7].
  // Issued after the list's first chunks (whose first use waits only for
  // those) and awaited together with the first stage copies.
  bf16x8 qf[KS];
  {
    const uint16_t* qp =
        p.q + (int64_t)b * p.qs0 + (int64_t)qrow * p.qs1 + (int64_t)h * p.qs2 + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
  }

  const uint16_t* kbase = p.k + (int64_t)b * p.ks0 + (int64_t)g * p.ks2;
  const uint16_t* vbase = p.v + (int64_t)b * p.vs0 + (int64_t)g * p.vs2;
  Copy kcopy, vcopy;
  kcopy.init(p.ks1, lane, wave);
  vcopy.init(p.vs1, lane, wave);
  // LDS: K stages 0, 1 then V stages 0, 1; this wave copies rows RPW wave ..
  const uint32_t smem_addr =
      (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint16_t*)smem);
  const uint32_t wcopy = (uint32_t)(wave * RPW * D * 2);
  auto k_stage = [&](int s) { return smem_addr + (uint32_t)(s * STAGE * 2) + wcopy; };
  auto v_stage = [&](int s) { return smem_addr + (uint32_t)((2 + s) * STAGE * 2) + wcopy; };

  // Listed block n. Entries outside [0, NK) are copied from block 0 (always
  // in bounds) with no real key, which gives them zero weight.
  auto block_of = [&](int n_pos) -> int {
    int n = n_pos + n_first;
    if (n >= nblk) n -= nblk;
    if constexpr (DENSE) {
      return n < p.n_forced ? n : p.n_prefix_blocks + (n - p.n_forced);
    } else {
      return __builtin_amdgcn_readlane(lw_cur, n_pos & 63);  // n_pos lies in chunk lw_c
    }
  };
  // Real keys of block j form a prefix [0, nvalid) of the block: segments
  // are block aligned and padding follows the real keys of each segment.
  auto nvalid_of = [&](int j) -> int {
    if (j < 0 || j >= p.nk) return 0;
    const int s0 = j * BK;
    const int seg_end =
        (s0 < p.kv_prefix_len) ? p.kv_prefix_valid : p.kv_prefix_len + p.kv_suffix_valid;
    return min(max(seg_end - s0, 0), BK);
  };
  // First HBM row copied by this wave for stage x of block j.
  auto copy_row_of = [&](int j, int x) -> int64_t {
    return ((j < 0 || j >= p.nk) ? 0 : (int64_t)j * BK) + (x % SPB) * 64 + wave * RPW;
  };
  // Real keys among this wave's 32 keys of stage x of a block with nv real keys.
  auto nvs_of = [&](int nv, int x) { return min(max(nv - (x % SPB) * 64 - kh * 32, 0), 32); };
  // Rank among the real keys of the first of this wave's 32 keys of stage x
  // of block j (causal mode; blocks are segment aligned and real keys lead
  // each segment).
  auto rank0_of = [&](int j, int x) {
    const int k0 = j * BK + (x % SPB) * 64 + 32 * kh;
    return j < p.n_prefix_blocks ? k0 : p.kv_prefix_valid + (k0 - p.kv_prefix_len);
  };

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  const float sl2 = p.scale_log2;

  // LDS element offsets (within a stage) that do not depend on the stage.
  const int sw = swz<CPR>(col);  // swizzle of K row 32 kh + col
  int koffs[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koffs[ks] = (32 * kh + col) * D + (((2 * ks + half) ^ sw) << 3);
  const int g16 = lane >> 4, j16 = lane & 15, tq = j16 >> 2, q4 = j16 & 3;
  int voffs[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int d = dt * 32 + 16 * (g16 & 1) + 4 * q4;
      const int row = 8 * c2 + 4 * half + tq;  // + 32 kh + 16 per key step
      voffs[dt][c2] = (32 * kh + row) * D + (((d >> 3) ^ swz<CPR>(row)) << 3) + (d & 7);
    }

  // Softmax state of this lane's query row over this wave's keys.
  float m_run = -__builtin_inff();  // reference max (log2 units)
  float m_use = 0.0f;               // m_run, or 0 while it is -inf
  float alpha = 1.0f;
  float lsum = 0.0f;                // this lane's part of the row sum, relative to m_use
  bool need = false;
  // Keys of the wave's 32 at or past `nvs` are padding. In causal mode key
  // kk also has rank rank0 + kk, and row qrow keeps ranks <= qrow + causal_off.
  auto mask = [&](f32x16& sd, int nvs, int rank0) {
    int lim = nvs;      // this lane keeps keys [0, lim)
    bool any = nvs < 32;
    if constexpr (CAUSAL) {
      lim = min(nvs, qrow + p.causal_off - rank0 + 1);
      any = any || (row0 + 32 * qh + p.causal_off - rank0 + 1 < 32);  // the wave's first row
    }
    if (any) {  // only stages that hold padding or cross the diagonal (uniform branch)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = (r >> 2) * 8 + half * 4 + (r & 3);
        sd[r] = key < lim ? sd[r] : -__builtin_inff();
      }
    }
  };
  // Reference update from the lane's partial row maximum of a fresh S.
  auto prep_tail = [&](float mxl) {
    // When no lane's partial maximum clears its row's reference by the slack,
    // neither does any row maximum and nothing changes (the usual case after
    // the first stages): the cross-lane step is skipped.
    float mx = -__builtin_inff();
    if (__builtin_amdgcn_ballot_w64(mxl * sl2 > m_run + kRescaleSlack) != 0)
      mx = max_with_other_half(mxl) * sl2;
    const bool moves = mx > m_run + kRescaleSlack;
    // While the reference is -inf no key has contributed: nothing to rescale.
    need = moves && m_run != -__builtin_inff();
    const float e_alpha = __builtin_amdgcn_exp2f(m_run - mx);
    alpha = need ? e_alpha : 1.0f;
    m_run = moves ? mx : m_run;
    m_use = (m_run == -__builtin_inff()) ? 0.0f : m_run;
  };
  auto prep = [&](const f32x16& sd) {
    float mxl = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; r += 2) mxl = __builtin_fmaxf(mxl, __builtin_fmaxf(sd[r], sd[r + 1]));
    prep_tail(mxl);
  };

  // Blocks around the current stage u (in block n = u / SPB):
  // (j0, nv0) block n, (j1, nv1) block n + 1, (j2, nv2) block n + 2.
  int j0 = -1, nv0 = 0, j1 = -1, nv1 = 0, j2 = -1, nv2 = 0;
  f32x16 sA, sB;

  if (nst > 0) {
    j0 = block_of(0);
    nv0 = nvalid_of(j0);
    if (nblk > 1) {
      j1 = block_of(1);
      nv1 = nvalid_of(j1);
    }
    kcopy.issue(kbase + copy_row_of(j0, 0) * p.ks1, k_stage(0));
    vcopy.issue(vbase + copy_row_of(j0, 0) * p.vs1, v_stage(0));
    if (nst > 1) {
      const int jn = (SPB == 1) ? j1 : j0;
      kcopy.issue(kbase + copy_row_of(jn, 1) * p.ks1, k_stage(1));
    }
    wait_vmcnt<0>();
    lds_barrier();
#pragma unroll
    for (int r = 0; r < 16; ++r) sA[r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(smem + koffs[ks]);
      sA = mfma(a, qf[ks], sA);
    }
    mask(sA, nvs_of(nv0, 0), CAUSAL ? rank0_of(j0, 0) : 0);
    prep(sA);
  }

  // One pipeline step on stage u. KP: the K stage read in this step (that of
  // stage u + 1); VP: the V stage (that of stage u). Copies issued here: V of
  // u + 1 into V stage VP ^ 1 and K of u + 2 into K stage KP ^ 1; both were
  // last read in the previous step, which every wave has left at the barrier.
  auto step = [&](auto kp_c, auto vp_c, int u, f32x16& s_cur, f32x16& s_nxt) {
    constexpr int KP = decltype(kp_c)::value;
    constexpr int VP = decltype(vp_c)::value;
    const bool last_sub = (u % SPB) == SPB - 1;
    const int n = u / SPB;
    if (last_sub) {
      if constexpr (!DENSE) {
        if (n + 2 < nblk && ((n + 2) & 63) == 0) {
          lw_cur = lw_next;
          ++lw_c;
          lw_next = load_chunk(lw_c + 1);
        }
      }
      j2 = (n + 2 < nblk) ? block_of(n + 2) : -1;
      nv2 = (n + 2 < nblk) ? nvalid_of(j2) : 0;
    }
    // ---- the step's single synchronisation point.
    wait_vmcnt<0>();
    lds_barrier();
    // Past the end of the list the copies still run (their slots are never
    // read again, or only by the masked dummy product) but read this head's
    // first rows, which are always in bounds: no branch per copy.
    const bool v_next = u + 1 < nst, k_next = u + 2 < nst;
    const uint16_t* v_rows =
        v_next ? vbase + copy_row_of((SPB == 1 || last_sub) ? j1 : j0, u + 1) * p.vs1
               : vbase + (int64_t)wave * RPW * p.vs1;
    const uint16_t* k_rows =
        k_next ? kbase + copy_row_of((SPB == 1) ? j2 : j1, u + 2) * p.ks1
               : kbase + (int64_t)wave * RPW * p.ks1;
    const uint16_t* kb = smem + KP * STAGE;
    uint16_t* vb = smem + (2 + VP) * STAGE;
    const int nvs = nvs_of(nv0, u);
    if (nvs < 32) {
      // Padded keys get weight 0, but 0 * NaN is NaN: clear their V rows
      // (both waves of this key half write the same zeros).
      uint4* vz = reinterpret_cast<uint4*>(vb + (32 * kh + nvs) * D);
      const int nz = (32 - nvs) * D / 8;
      for (int e = lane; e < nz; e += 64) vz[e] = make_uint4(0, 0, 0, 0);
    }
    // Lazy rescale of the running output (rare after the first stages).
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }

    // ---- (a) S[u+1] = K Q^T || exponentials of P[u] || V^T reads || copies.
    bf16x8 pf[2];
    bf16x4 vf[2][DT][2];
    constexpr int EXP_PER = 16 / KS;  // exponentials per MFMA slot
    constexpr int NVRD = 2 * DT * 2;  // V^T reads of the step
    constexpr int VRD_PER = NVRD / KS;
    static_assert(NVRD % KS == 0, "V reads per slot");
    bf16x8 kf[3];
    kf[0] = *reinterpret_cast<const bf16x8*>(kb + koffs[0]);
    kf[1] = *reinterpret_cast<const bf16x8*>(kb + koffs[1]);
#pragma unroll
    for (int r = 0; r < 16; ++r) s_nxt[r] = 0.0f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      if (k + 2 < KS) kf[(k + 2) % 3] = *reinterpret_cast<const bf16x8*>(kb + koffs[k + 2]);
      s_nxt = mfma(kf[k % 3], qf[k], s_nxt);
      // The copy instructions spread evenly over the slots (V of u + 1, then
      // K of u + 2).
      static_assert(KS % (2 * Copy::NL) == 0, "copy slots");
      constexpr int CEVERY = KS / (2 * Copy::NL);
      if (k % CEVERY == 0) {
        const int c = k / CEVERY;
        if (c < Copy::NL) {
          vcopy.issue_one(c, v_rows, v_stage(VP ^ 1));
        } else {
          kcopy.issue_one(c - Copy::NL, k_rows, k_stage(KP ^ 1));
        }
      }
#pragma unroll
      for (int x = 0; x < EXP_PER; ++x) {
        const int r = k * EXP_PER + x;
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r], sl2, -m_use));
        // Pin the exponential to this slot: without it the compiler sinks
        // the softmax below the masking branch, after every QK^T MFMA.
        asm volatile("" : "+v"(e));
        lsum += e;
        pf[r / 8][r % 8] = (__bf16)e;
      }
#pragma unroll
      for (int x = 0; x < VRD_PER; ++x) {
        const int idx = k * VRD_PER + x;
        const int ks2 = idx / (DT * 2), dt = (idx / 2) % DT, c2 = idx % 2;
        vf[ks2][dt][c2] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(vb + 16 * ks2 * D + voffs[dt][c2]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // With no next stage, S[u+1] is a dummy product and every key of it
    // counts as padding, which leaves the softmax state unchanged.
    const int nvs_next = (u + 1 < nst) ? nvs_of((SPB == 1 || last_sub) ? nv1 : nv0, u + 1) : 0;
    mask(s_nxt, nvs_next,
         CAUSAL ? rank0_of((SPB == 1 || last_sub) ? j1 : j0, u + 1) : 0);
    // ---- (b) O += V^T P[u]^T || row max of S[u+1].
    float mxl = -__builtin_inff();
    constexpr int NPV = 2 * DT;
#pragma unroll
    for (int sl = 0; sl < NPV; ++sl) {
      const int ks2 = sl / DT, dt = sl % DT;
      const bf16x8 av =
          __builtin_shufflevector(vf[ks2][dt][0], vf[ks2][dt][1], 0, 1, 2, 3, 4, 5, 6, 7);
      o[dt] = mfma(av, pf[ks2], o[dt]);
#pragma unroll
      for (int it = sl * 8 / NPV; it < (sl + 1) * 8 / NPV; ++it) {
        mxl = __builtin_fmaxf(mxl, __builtin_fmaxf(s_nxt[2 * it], s_nxt[2 * it + 1]));
        asm volatile("" : "+v"(mxl));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    prep_tail(mxl);

    if (last_sub) {
      j0 = j1;
      nv0 = nv1;
      j1 = j2;
      nv1 = nv2;
    }
  };

  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  // Two stages per loop turn so that the LDS stages and the S registers
  // alternate statically.
  for (int u = 0; u < nst; u += 2) {
    step(C1{}, C0{}, u, sA, sB);
    if (u + 1 < nst) step(C0{}, C1{}, u + 1, sB, sA);
  }

  // ---- epilogue: merge the two key halves of each query half. Wave
  // (qh, kh) finishes output tiles [kh DT/2, (kh + 1) DT/2) and hands the
  // other half of its tiles, its reference and its row sum to wave
  // (qh, 1 - kh) through LDS (free once every wave has left the loop).
  const float ltot = sum_with_other_half(lsum);
  constexpr int HT = DT / 2;   // output tiles finished per wave
  constexpr int XR = HT * 16;  // accumulator registers handed over
  wait_vmcnt<0>();  // the last steps' copies land before the LDS is reused
  lds_barrier();
  float* xo = reinterpret_cast<float*>(smem) + wave * (XR + 2) * 64;
  const float* yo = reinterpret_cast<const float*>(smem) + (wave ^ 1) * (XR + 2) * 64;
  auto hand_over = [&](auto first_c) {
    constexpr int F = decltype(first_c)::value;
#pragma unroll
    for (int x = 0; x < HT; ++x)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(x * 16 + r) * 64 + lane] = o[F + x][r];
  };
  if (kh == 0)
    hand_over(std::integral_constant<int, HT>{});
  else
    hand_over(std::integral_constant<int, 0>{});
  xo[XR * 64 + lane] = m_use;
  xo[(XR + 1) * 64 + lane] = ltot;
  lds_barrier();
  const float m2 = yo[XR * 64 + lane], l2 = yo[(XR + 1) * 64 + lane];
  const bool e1 = ltot > 0.0f, e2 = l2 > 0.0f;
  const float mm = __builtin_fmaxf(e1 ? m_use : -__builtin_inff(), e2 ? m2 : -__builtin_inff());
  const float a1 = e1 ? __builtin_amdgcn_exp2f(m_use - mm) : 0.0f;
  const float a2 = e2 ? __builtin_amdgcn_exp2f(m2 - mm) : 0.0f;
  const float l_run = ltot * a1 + l2 * a2;
  const bool row_ok = qrow < p.q_valid && l_run > 0.0f;
  const float inv = row_ok ? 1.0f / l_run : 0.0f;
  const float c1 = a1 * inv, c2 = a2 * inv;
  // O^T lane layout: query col, d = dt*32 + (r/4)*8 + half*4 + r%4.
  uint16_t* op = p.o + (int64_t)b * p.os0 + (int64_t)qrow * p.os1 + (int64_t)h * p.os2;
  auto finish = [&](auto first_c) {
    constexpr int F = decltype(first_c)::value;
#pragma unroll
    for (int x = 0; x < HT; ++x)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = rg * 4 + e;
          const float v = o[F + x][r] * c1 + yo[(x * 16 + r) * 64 + lane] * c2;
          vv[e] = (__bf16)(row_ok ? v : 0.0f);
        }
        *reinterpret_cast<bf16x4*>(op + (F + x) * 32 + rg * 8 + half * 4) = vv;
      }
  };
  if (kh == 0)
    finish(std::integral_constant<int, 0>{});
  else
    finish(std::integral_constant<int, HT>{});
  if (p.lse != nullptr && kh == 0 && half == 0) {
    const float lse = row_ok ? (mm + __builtin_log2f(l_run)) * 0.69314718055994531f
                             : -__builtin_inff();
    p.lse[((int64_t)b * p.hq + h) * p.q_len + qrow] = lse;
  }
}

// LDS of a workgroup: the four stages, or the epilogue's hand-over area if
// that is larger (eight waves at head dim 128).
template <int D, int NQG>
constexpr int smem_elems() {
  constexpr int stages = 4 * 64 * D;
  constexpr int handover = 2 * NQG * ((D / 64) * 16 + 2) * 64 * 2;  // floats -> bf16 units
  return stages > handover ? stages : handover;
}

// Waves per SIMD: two at head_dim 128 (up to 256 VGPRs each), three at
// head_dim 64 (up to 168; the kernel needs about 160 there).
template <int D>
constexpr int waves_per_simd() { return D == 64 ? 3 : 2; }

template <int D, int BK, int NQG, int MODE>
__global__ void __launch_bounds__(128 * NQG)
__attribute__((amdgpu_waves_per_eu(waves_per_simd<D>(), waves_per_simd<D>())))
attn_fwd_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[smem_elems<D, NQG>()];
  attn_fwd_body<D, BK, NQG, MODE>(p, smem);
}

template <int D, int BK, int NQG, int MODE>
hipError_t launch_one(const AttnParams& p, hipStream_t stream) {
  const int grid =
      p.head_sync ? p.batch * p.hkv * 8 * ((p.nq * p.group * p.qparts + 7) / 8) : p.n_wg;
  hipLaunchKernelGGL((attn_fwd_kernel<D, BK, NQG, MODE>), dim3(grid), dim3(128 * NQG), 0, stream,
                     p);
  return hipGetLastError();
}

template <int D, int BK, int NQG>
hipError_t launch_mode(const AttnParams& p, int mode, hipStream_t stream) {
  switch (mode) {
    case kSparse: return launch_one<D, BK, NQG, kSparse>(p, stream);
    case kDense: return launch_one<D, BK, NQG, kDense>(p, stream);
    default: return launch_one<D, BK, NQG, kCausal>(p, stream);
  }
}

template <int D, int NQG>
hipError_t launch_geom(const AttnParams& p, int bk, int mode, hipStream_t stream) {
  if (bk == 64) return launch_mode<D, 64, NQG>(p, mode, stream);
  return launch_mode<D, 128, NQG>(p, mode, stream);
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, int head_dim, int block_q, int block_k, int mode,
                            hipStream_t stream) {
  if (p.n_wg == 0) return hipSuccess;
  if (mode != kSparse && mode != kDense && mode != kCausal) return hipErrorInvalidValue;
  // One workgroup per query block: 4 waves for 64 rows, 8 waves for 128 rows;
  // 256-row blocks run as two 128-row workgroups (p.qparts = 2).
  if (head_dim == 128)
    return block_q == 64 ? launch_geom<128, 2>(p, block_k, mode, stream)
                         : launch_geom<128, 4>(p, block_k, mode, stream);
  return block_q == 64 ? launch_geom<64, 2>(p, block_k, mode, stream)
                       : launch_geom<64, 4>(p, block_k, mode, stream);
}

}  // namespace bsattn
