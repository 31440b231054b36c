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
// fewer than 168 and a SIMD runs three.
//
// What the main loop issues per wave and 64-key stage is kept to what the
// matrix products need: on gfx950 every vector, scalar and LDS instruction a
// SIMD issues between its matrix instructions costs matrix-core time, and so
// does every wait on memory. Under this load the chip also runs at its power
// limit, so every byte moved (stage copies through L2, LDS operand reads)
// costs clock.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the K fragment (A operand)
//    comes from LDS, Q^T (B operand) stays in registers for the whole
//    kernel. Each lane owns one query row and half of the wave's 32 keys.
//  * Online softmax in fp32 in the log2 domain, the scale folded into the
//    exponential's FMA. A row's reference maximum moves only when a stage
//    maximum exceeds it by more than 2^8 (lazy rescale); the per-stage test
//    is one compare against a precomputed threshold, and everything else
//    (the cross-lane maximum, the rescale of the running output) runs only
//    when some lane trips it, which after the first stages is rare. Row sums
//    add the fp32 probabilities in two independent chains.
//  * O^T = V^T P^T with the same MFMA: P^T is the S^T accumulator converted
//    to bf16 (the contraction over keys is order-free, so the key order of
//    the accumulator layout is reused for V); V^T fragments come from the
//    row-major V tile through ds_read_b64_tr_b16.
//  * Inside a wave the QK^T MFMAs of the next stage are interleaved with the
//    exponentials of the current one, and the PV MFMAs with the row maxima
//    of the next.
//  * K and V stages move HBM -> LDS with buffer_load_dwordx4 ... lds (no
//    VGPR staging): the buffer resource of the (batch, KV head) and each
//    lane's offset are fixed, the stage enters as one scalar byte offset,
//    and M0 (the LDS destination) is set once per stage buffer.
//    Rows are XOR-swizzled in 16-byte chunks so the K row reads and the V
//    transpose reads hit distinct banks. K and V each have a ring of R
//    stages in LDS and are copied R - 1 stages ahead of their use, so a
//    stage's wait leaves the copies of the R - 2 newest stages in flight:
//    a copy has R - 1 stages of time to land. One workgroup barrier per
//    stage.
//  * The block list is read 64 entries per vector load; each entry becomes a
//    descriptor (first key row, real keys in the block) once, and a stage
//    takes its descriptor with one v_readlane.
//  * Workgroups are renumbered so that each XCD works through a contiguous
//    range of (KV head, query head, query block), keeping that range's K/V
//    tiles in the XCD's L2.

#include <type_traits>
#include <utility>

#include "internal.h"

namespace bsattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

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
// across it; their completion is awaited explicitly with wait_vmcnt. The
// empty asm statements keep the compiler from moving memory operations
// (the copies included) across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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

// Stages of K (and of V) in LDS: two of each. A 64-row workgroup shares its
// CU with another one and has 64 KB of LDS. A 128-row workgroup has the
// CU's LDS to itself and could hold four stages of each, but copying three
// stages ahead measured 3-9 % slower than one (on gfx950 these copies cost
// through the power they draw, not through their latency). The loop is
// unrolled R stages deep (a ring of three would need six, and the longer
// live ranges then spill the Q fragments).
template <int D, int NQG>
constexpr int kv_ring() { return 2; }

// Work split inside each XCD pair. Under the power limit the odd-numbered
// XCDs run at a lower shader clock than the even ones (0.95-0.97 of it on
// every box measured, in every workload that keeps the chip busy), so with
// equal shares the even XCDs finish early and idle. A launch in which every
// XCD runs at least 32 rounds of its resident workgroups gives the even XCD
// of each pair 50.6 % of the pair's work (the best of the shares timed at
// 48k; larger ones cost more in L2 locality than they save), in the
// contiguous order and, per KV head, in the head-synchronous one. A shorter
// launch splits evenly: a larger share that adds a partial round costs more
// than the clocks (8 rounds at dense 8k: 4.8 % slower). The split depends
// only on the launch's shape, so results stay bitwise reproducible.
constexpr int kEvenShare16 = 33161;  // 0.506 x 65536

__host__ __device__ __forceinline__ int even_count(int pair_work, int share16) {
  return (int)(((int64_t)pair_work * share16 + 32768) >> 16);
}

template <int D, int NQG>
int pair_split(const AttnParams& p) {
  constexpr int resident = NQG == 2 ? (D == 64 ? 3 : 2) : 1;  // workgroups per CU
  const int per_xcd = (p.n_wg + 7) / 8;
  const bool long_launch = per_xcd >= 32 * 32 * resident;  // 32 rounds on 32 CUs
  return (D == 128 && long_launch) ? kEvenShare16 : 32768;
}

template <int D, int BK, int NQG, int MODE>
__device__ __forceinline__ void attn_fwd_body(const AttnParams& p, uint16_t* __restrict__ smem) {
  constexpr bool DENSE = MODE != kSparse;    // the list is every non-empty block
  constexpr bool CAUSAL = MODE == kCausal;   // ... cut to the causal range
  constexpr int CPR = D / 8;     // 16-byte chunks per K/V row
  constexpr int KS = D / 16;     // MFMA k-steps over D (QK^T MFMAs per stage)
  constexpr int DT = D / 32;     // output 32-row tiles over D
  constexpr int SPB = BK / 64;   // 64-key stages per block
  constexpr int STAGE = 64 * D;  // elements of one K or V stage
  static_assert(SPB == 1 || SPB == 2, "block_k 64 or 128");
  constexpr int NW = 2 * NQG;    // waves: NQG query groups of 32 rows x 2 key halves
  constexpr int RPW = 64 / NW;   // stage rows copied by each wave
  constexpr int RPI = 64 / CPR;  // rows moved by one copy instruction (64 lanes x 16 bytes)
  constexpr int NL = RPW / RPI;  // copy instructions per wave for one K (or V) stage
  static_assert(NL >= 1 && NL * RPI == RPW, "rows per wave");
  constexpr int R = kv_ring<D, NQG>();   // K and V stages in LDS (copied R - 1 stages ahead)
  static_assert(R == 2 || R == 4, "rings of two or four stages");
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

  // Workgroup w runs on XCD w % 8. The work is the (batch, KV head,
  // head-in-group, query block, part) order; a query block of more than 128
  // rows is split into parts of 32 NQG rows, one workgroup each, reading the
  // same list. Each XCD takes a contiguous range of that order, so the
  // workgroups it runs together are adjacent query blocks of one query head,
  // whose lists are the most alike (on the 48k inputs adjacent blocks of a
  // head share 61 % of their lists, the heads of a group 34 %), and read
  // many of the same K/V blocks through its L2. When the K/V of all heads would not fit in the 256 MB last-level
  // cache together, the XCDs instead split every (batch, KV head) eight ways
  // and move through the KV heads in step, so only one head's K/V is live;
  // the grid is then padded to a multiple of eight per (batch, KV head).
  const int w = blockIdx.x;
  const int xcd = w & 7, kx = w >> 3;
  int lin, bg;
  if (p.head_sync && p.even_share16 == 32768) {
    const int tot = p.nq * p.group * p.qparts;  // workgroups per (batch, KV head)
    const int per = (tot + 7) >> 3;
    bg = kx / per;
    lin = xcd * per + kx % per;
    if (lin >= tot) return;  // padding: the whole workgroup leaves before any barrier
  } else if (p.head_sync) {
    // The same, with each (batch, KV head)'s work split between the XCDs of
    // a pair as in the contiguous order below.
    const int tot = p.nq * p.group * p.qparts;
    const int q4 = tot >> 2, r4 = tot & 3;
    const int per = even_count(q4 + (r4 ? 1 : 0), p.even_share16);  // per head and XCD
    const int j = xcd >> 1;
    const int pj = q4 + (j < r4 ? 1 : 0);
    const int ej = even_count(pj, p.even_share16);
    bg = kx / per;
    const int loc = kx % per;
    if (loc >= ((xcd & 1) ? pj - ej : ej)) return;  // leaves before any barrier
    lin = j * q4 + min(j, r4) + ((xcd & 1) ? ej : 0) + loc;
  } else {
    // The work goes to the four XCD pairs as evenly as possible, and within
    // a pair the even XCD takes even_share16 / 65536 of it (pair_split).
    // The grid gives every XCD as many workgroups as the largest share; an
    // odd XCD's surplus ones have no work.
    const int nwg = p.n_wg, q4 = nwg >> 2, r4 = nwg & 3;
    const int j = xcd >> 1;
    const int pj = q4 + (j < r4 ? 1 : 0);
    const int ej = even_count(pj, p.even_share16);
    const int start = j * q4 + min(j, r4) + ((xcd & 1) ? ej : 0);
    if (kx >= ((xcd & 1) ? pj - ej : ej)) return;  // leaves before any barrier
    const int all = start + kx;
    const int tot = p.nq * p.group * p.qparts;
    bg = all / tot;
    lin = all % tot;
  }
  const int part = lin % p.qparts;
  int t = lin / p.qparts;
  const int hig = t / p.nq;
  const int i = t % p.nq;
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
    nblk = min(max(__builtin_amdgcn_readfirstlane(p.cnt[row_id]), 0), p.idx_row_stride);
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
  // The half-lifetime lag builds up over the first rounds: both cohorts of
  // round 0 start together, and the second cohort's lag grows to about half
  // a lifetime by round 6 (measured on XCD 0 at 48k: 0, 13, 20, 23, 27, 29
  // and 30 sixty-fourths of a lifetime in rounds 0-6). At head_dim 128 the
  // second cohort of round r starts kLead64[min(r, 7)] sixty-fourths into
  // its list: 0, 16, 24, 28, 30, 31, 32, 32, a little ahead of the lags,
  // which timed best among the tables tried.
  const int cohort = (w >> 8) % (D == 64 ? 3 : 2);  // (w / 8) / 32: cohorts of 32 per XCD
  int n_first = (NQG == 2) ? (cohort * nblk) / (D == 64 ? 3 : 2) : 0;
  if constexpr (NQG == 2 && D == 128) {
    constexpr uint64_t kLead64 = 0x8207de718400ull;  // 6 bits per round, round 0 lowest
    const int rnd = min(kx >> 6, 7);                 // round of 64 workgroups on the XCD
    n_first = cohort ? ((int)((kLead64 >> (6 * rnd)) & 63) * nblk) >> 6 : 0;
  }

  // Block j as a descriptor: (first key row << 8) | real keys in the block,
  // 0 for an entry outside [0, NK) (copied from block 0, every key masked).
  // Real keys of a block form a prefix of it: segments are block aligned and
  // padding follows the real keys of each segment.
  auto desc_of_block = [&](int j) -> int {
    const int s0 = j * BK;
    const int seg_end =
        (s0 < p.kv_prefix_len) ? p.kv_prefix_valid : p.kv_prefix_len + p.kv_suffix_valid;
    const int nv = min(max(seg_end - s0, 0), BK);
    return (j < 0 || j >= p.nk) ? 0 : ((s0 << 8) | nv);
  };
  // The list, 64 positions at a time: lane l of lw_cur holds the descriptor
  // of list position 64 c + l (after the rotation) for the current chunk c;
  // lw_raw holds the raw entries of chunk c + 1, loaded a whole chunk ahead
  // (unconditionally, from a position clamped into the list, so that the
  // load lands in its own register and nothing waits for it until the
  // chunk is used; positions past the end are dropped at that point).
  int lw_cur = 0, lw_raw = -1, lw_c = 0;
  auto load_chunk = [&](int c) -> int {
    int n = min(c * 64 + lane, nblk - 1) + n_first;
    if (n >= nblk) n -= nblk;
    return idx_row[n];
  };
  auto chunk_desc = [&](int raw, int c) {
    return desc_of_block(c * 64 + lane < nblk ? raw : -1);
  };
  if constexpr (!DENSE) {
    if (nblk > 0) {
      lw_cur = chunk_desc(load_chunk(0), 0);
      lw_raw = load_chunk(1);
    }
  }
  // Descriptor of list position n_pos (positions are asked for in order).
  auto block_desc = [&](int n_pos) -> int {
    if constexpr (DENSE) {
      int n = n_pos + n_first;
      if (n >= nblk) n -= nblk;
      return desc_of_block(n < p.n_forced ? n : p.n_prefix_blocks + (n - p.n_forced));
    } else {
      if ((n_pos >> 6) != lw_c) {  // next chunk (uniform, once per 64 positions)
        ++lw_c;
        lw_cur = chunk_desc(lw_raw, lw_c);
        lw_raw = load_chunk(lw_c + 1);
      }
      return __builtin_amdgcn_readlane(lw_cur, n_pos & 63);
    }
  };

  // Q^T fragments (B operand): the lane holds q[qrow][16 ks + 8 half .. +7].
  bf16x8 qf[KS];
  {
    const uint16_t* qp =
        p.q + (int64_t)b * p.qs0 + (int64_t)qrow * p.qs1 + (int64_t)h * p.qs2 + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
  }

  // Copies: one buffer resource per (batch, KV head) for K and for V, a fixed
  // per-lane byte offset per copy instruction (row within the stage and
  // swizzled chunk), and the stage's first key row as a scalar byte offset.
  // Copy instruction `it` of a stage writes LDS 1 KB further on than copy
  // it - 1; that step is the instruction's immediate offset, which moves the
  // LDS and the memory address alike, so it is taken back out of the lane's
  // memory offset and M0 is set once per stage buffer. The resources start
  // (NL - 1) KB before the head's first row (and reach as much further), so
  // that the lane offsets stay non-negative for any row stride; every address
  // a copy reads is still inside the head's rows.
  static_assert(NL <= 4, "copy offsets fit the 12-bit immediate");
  constexpr uint32_t SHIFT = (NL - 1) * 1024;
  const uintptr_t kbase = (uintptr_t)(p.k + (int64_t)b * p.ks0 + (int64_t)g * p.ks2);
  const uintptr_t vbase = (uintptr_t)(p.v + (int64_t)b * p.vs0 + (int64_t)g * p.vs2);
  const auto krsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(kbase - SHIFT), 0,
                                                       p.k_span_bytes + SHIFT, 0x00020000);
  const auto vrsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(vbase - SHIFT), 0,
                                                       p.v_span_bytes + SHIFT, 0x00020000);
  const int krow_b = (int)p.ks1 * 2, vrow_b = (int)p.vs1 * 2;  // bytes per key row
  int kvoff[NL], vvoff[NL];
#pragma unroll
  for (int it = 0; it < NL; ++it) {
    const int row = wave * RPW + it * RPI + lane / CPR;  // row within the stage
    const int gch = (lane % CPR) ^ swz<CPR>(row);         // chunk this lane's LDS slot holds
    kvoff[it] = row * krow_b + gch * 16 + (int)SHIFT - it * 1024;
    vvoff[it] = row * vrow_b + gch * 16 + (int)SHIFT - it * 1024;
  }
  lds_u16* const lds = (lds_u16*)smem;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  // LDS: K stages 0 .. R - 1, then V stages 0 .. R - 1. A copy instruction writes
  // 64 lanes x 16 bytes from M0 + 1 KB it on, rows RPW wave + RPI it .. of its
  // stage. Copy 0 of a stage buffer sets M0 (nothing else here uses it) and
  // copies 1 .. NL - 1 follow it with no other copy in between.
  // The copies are issued from inline assembly: the compiler then neither
  // counts them nor orders LDS reads behind them (it cannot tell that they
  // write other stages than the ones being read), so every read of a stage
  // is preceded by an explicit wait_vmcnt and a workgroup barrier.
  auto copy_one = [&](auto it_c, const __amdgpu_buffer_rsrc_t& rsrc, uint32_t m0, int voff, int soff) {
    constexpr int IT = decltype(it_c)::value;
    if constexpr (IT == 0) {
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                   :
                   : "s"(m0), "v"(voff), "s"(rsrc), "s"(soff)
                   : "m0");
    } else {
      asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds"
                   :
                   : "v"(voff), "s"(rsrc), "s"(soff), "i"(IT * 1024));
    }
  };
  auto copy_k = [&](auto kb_c, auto it_c, int row) {
    constexpr int KB = decltype(kb_c)::value;
    constexpr int IT = decltype(it_c)::value;
    copy_one(it_c, krsrc, lds_addr + (uint32_t)((KB * STAGE + (wave * RPW) * D) * 2),
             kvoff[IT], row * krow_b);
  };
  auto copy_v = [&](auto vb_c, auto it_c, int row) {
    constexpr int VB = decltype(vb_c)::value;
    constexpr int IT = decltype(it_c)::value;
    copy_one(it_c, vrsrc, lds_addr + (uint32_t)(((R + VB) * STAGE + (wave * RPW) * D) * 2),
             vvoff[IT], row * vrow_b);
  };
  // Copy `it` of an unrolled loop (a constant after unrolling) as a
  // compile-time index.
  auto copy_k_at = [&](auto kb_c, int it, int row) {
    if constexpr (NL > 0) if (it == 0) copy_k(kb_c, std::integral_constant<int, 0>{}, row);
    if constexpr (NL > 1) if (it == 1) copy_k(kb_c, std::integral_constant<int, 1 % NL>{}, row);
    if constexpr (NL > 2) if (it == 2) copy_k(kb_c, std::integral_constant<int, 2 % NL>{}, row);
    if constexpr (NL > 3) if (it == 3) copy_k(kb_c, std::integral_constant<int, 3 % NL>{}, row);
  };
  auto copy_v_at = [&](auto vb_c, int it, int row) {
    if constexpr (NL > 0) if (it == 0) copy_v(vb_c, std::integral_constant<int, 0>{}, row);
    if constexpr (NL > 1) if (it == 1) copy_v(vb_c, std::integral_constant<int, 1 % NL>{}, row);
    if constexpr (NL > 2) if (it == 2) copy_v(vb_c, std::integral_constant<int, 2 % NL>{}, row);
    if constexpr (NL > 3) if (it == 3) copy_v(vb_c, std::integral_constant<int, 3 % NL>{}, row);
  };

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  const float sl2 = p.scale_log2;
  const float inv_sl2 = 1.0f / sl2;

  // LDS element offsets (within a stage) that do not depend on the stage.
  const int sw = swz<CPR>(col);  // swizzle of K row 32 kh + col
  int koffs[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koffs[ks] = (32 * kh + col) * D + (((2 * ks + half) ^ sw) << 3);
  // V^T reads: LDS byte address of the lane's fragment in V stage 0. The V
  // stages lie above the K ring, past 64 KB for the second one; the base is
  // hidden from the compiler's constant folding so that both stages (and
  // both key steps) are immediate offsets from these registers.
  const int g16 = lane >> 4, j16 = lane & 15, tq = j16 >> 2, q4 = j16 & 3;
  int vrd[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int d = dt * 32 + 16 * (g16 & 1) + 4 * q4;
      const int row = 8 * c2 + 4 * half + tq;  // + 32 kh + 16 per key step
      vrd[dt][c2] =
          (R * STAGE + (32 * kh + row) * D + (((d >> 3) ^ swz<CPR>(row)) << 3) + (d & 7)) * 2;
      asm volatile("" : "+v"(vrd[dt][c2]));
    }
  typedef __attribute__((address_space(3))) char lds_char;
  auto vread = [&](int vb_stage, int ks2, int dt, int c2) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4*)((lds_char*)lds + vrd[dt][c2] + (vb_stage * STAGE + 16 * ks2 * D) * 2));
  };

  // Softmax state of this lane's query row over this wave's keys.
  float m_run = -__builtin_inff();  // reference max (log2 units)
  float m_use = 0.0f;               // m_run, or 0 while it is -inf
  float thr = -__builtin_inff();    // raw-score threshold: (m_run + slack) / scale
  float lsum = 0.0f;                // this lane's part of the row sum, relative to m_use

  // Stage descriptors: first key row of the stage and real keys among its 64.
  // SUB is the stage's 64-key part of its block (x % SPB, a compile-time
  // value at every call). Stages past the end of the list keep the previous
  // descriptor: their copies land in buffers that are not read again.
  int blk_desc = 0;
  auto stage_desc = [&](auto sub_c, int x, int& row, int& nv) {
    constexpr int SUB = decltype(sub_c)::value;
    if (x < nst) {
      if constexpr (SUB == 0) blk_desc = block_desc(x / SPB);
      row = (blk_desc >> 8) + SUB * 64;
      nv = min(max((blk_desc & 255) - SUB * 64, 0), 64);
    }
  };

  // Keys of the wave's 32 at or past `nvs` are padding. In causal mode key
  // kk also has rank rank0 + kk, and row qrow keeps ranks <= qrow + causal_off.
  auto rank0_of = [&](int row) {
    const int k0 = row + 32 * kh;
    return k0 < p.kv_prefix_len ? k0 : p.kv_prefix_valid + (k0 - p.kv_prefix_len);
  };
  auto mask = [&](f32x16& sd, int nv, int row) {
    const int nvs = min(max(nv - 32 * kh, 0), 32);
    int lim = nvs;  // this lane keeps keys [0, lim)
    bool any = nvs < 32;
    if constexpr (CAUSAL) {
      const int rank0 = rank0_of(row);
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
  // Lazy rescale: `mxl` is the lane's maximum raw score over its keys of the
  // newest stage. One compare per stage; the rest only when a lane trips it.
  auto check_ref = [&](float mxl) {
    if (__builtin_amdgcn_ballot_w64(mxl > thr) != 0) {
      const float mx = max_with_other_half(mxl) * sl2;
      const bool moves = mx > m_run + kRescaleSlack;
      // While the reference is -inf no key has contributed: nothing to rescale.
      const float alpha =
          (moves && m_run != -__builtin_inff()) ? __builtin_amdgcn_exp2f(m_run - mx) : 1.0f;
      m_run = moves ? mx : m_run;
      m_use = (m_run == -__builtin_inff()) ? 0.0f : m_run;
      thr = (m_run + kRescaleSlack) * inv_sl2;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
  };
  auto row_max = [&](const f32x16& sd) {
    float mxl = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; r += 2) mxl = __builtin_fmaxf(mxl, __builtin_fmaxf(sd[r], sd[r + 1]));
    return mxl;
  };

  // Descriptors of the stages in the pipeline: before step u, index x holds
  // stage u + x (x < R); the step shifts them, so that index x then holds
  // stage u + 1 + x and the new stage u + R enters at index R - 1.
  int srow[R], snv[R];
#pragma unroll
  for (int x = 0; x < R; ++x) srow[x] = snv[x] = 0;
  f32x16 sbuf[2];

  // Outstanding copies a step's wait leaves in flight: those of the R - 2
  // newest steps (V, then K, NL instructions each).
  constexpr int INFLIGHT = (R - 2) * 2 * NL;
  if (nst > 0) {
    // Prologue: K of stages 0 .. R - 1 and V of stages 0 .. R - 2, in the
    // order K0 V0 K1 V1 ..., then S[0] once K0 has landed.
    stage_desc(std::integral_constant<int, 0>{}, 0, srow[0], snv[0]);
#pragma unroll
    for (int x = 1; x < R; ++x) {
      srow[x] = srow[x - 1];
      snv[x] = snv[x - 1];
      if (x % SPB == 0)
        stage_desc(std::integral_constant<int, 0>{}, x, srow[x], snv[x]);
      else
        stage_desc(std::integral_constant<int, 1 % SPB>{}, x, srow[x], snv[x]);
    }
    auto pro_copies = [&](auto x_c) {
      constexpr int X = decltype(x_c)::value;
#pragma unroll
      for (int it = 0; it < NL; ++it) copy_k_at(std::integral_constant<int, X>{}, it, srow[X]);
      if constexpr (X + 1 < R) {
#pragma unroll
        for (int it = 0; it < NL; ++it) copy_v_at(std::integral_constant<int, X>{}, it, srow[X]);
      }
    };
    pro_copies(std::integral_constant<int, 0>{});
    pro_copies(std::integral_constant<int, 1>{});
    if constexpr (R == 4) {
      pro_copies(std::integral_constant<int, 2 % R>{});
      pro_copies(std::integral_constant<int, 3 % R>{});
    }
    wait_vmcnt<(2 * R - 2) * NL>();  // K of stage 0
    lds_barrier();
#pragma unroll
    for (int r = 0; r < 16; ++r) sbuf[0][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(smem + koffs[ks]);
      sbuf[0] = mfma(a, qf[ks], sbuf[0]);
    }
    mask(sbuf[0], snv[0], srow[0]);
    check_ref(row_max(sbuf[0]));
  }

  // One pipeline step on stage u (step S of the unrolled loop, u % R == S).
  // K stage u + 1 is read from K buffer (S + 1) % R and V stage u from V
  // buffer S; the step copies K of u + R into K buffer S (last read for
  // S[u], in the previous step) and V of u + R - 1 into V buffer
  // (S + R - 1) % R (last read for PV of u - 1, in the previous step):
  // every wave has left the previous step at this step's barrier.
  int cur_nv = snv[0];  // real keys of the current stage
  auto run_step = [&](auto s_c, int u) {
    constexpr int S = decltype(s_c)::value;
    constexpr int KB = (S + 1) % R, VB = S;
    constexpr int KNEW = S, VNEW = (S + R - 1) % R;
    f32x16& s_cur = sbuf[S % 2];
    f32x16& s_nxt = sbuf[(S + 1) % 2];
    // Index x now holds stage u + 1 + x; stage u + R enters at R - 1.
#pragma unroll
    for (int x = 0; x + 1 < R; ++x) {
      srow[x] = srow[x + 1];
      snv[x] = snv[x + 1];
    }
    stage_desc(std::integral_constant<int, (S + R) % SPB>{}, u + R, srow[R - 1], snv[R - 1]);
    // ---- the step's single synchronisation point: V of u and K of u + 1
    // have landed (this wave's copies by the count, every wave's by the
    // barrier).
    wait_vmcnt<INFLIGHT>();
    lds_barrier();
    const uint16_t* kb = smem + KB * STAGE;
    uint16_t* vb = smem + (R + VB) * STAGE;
    {
      const int nvs = min(max(cur_nv - 32 * kh, 0), 32);
      if (nvs < 32) {
        // Padded keys get weight 0, but 0 * NaN is NaN: clear their V rows
        // (both waves of this key half write the same zeros).
        uint4* vz = reinterpret_cast<uint4*>(vb + (32 * kh + nvs) * D);
        const int nz = (32 - nvs) * D / 8;
        for (int e = lane; e < nz; e += 64) vz[e] = make_uint4(0, 0, 0, 0);
      }
    }

    // ---- (a) S[u+1] = K Q^T || exponentials of P[u] || V^T reads || copies.
    bf16x8 pf[2];
    // V^T fragments of the first 16 keys are read during (a), those of the
    // second 16 during the first PV products of (b) (into registers the
    // consumed S[u] leaves free).
    bf16x4 vf0[DT][2], vf1[DT][2];
    constexpr int EXP_PER = 16 / KS;  // exponentials per MFMA slot
    constexpr int NVRD = DT * 2;      // V^T reads of (a)
    constexpr int VRD_PER = NVRD / KS;
    static_assert(NVRD % KS == 0 && EXP_PER % 2 == 0, "slots");
    constexpr int NCOPY = 2 * NL;     // copy instructions of the step
    static_assert(KS % NCOPY == 0, "copy slots");
    constexpr int CEVERY = KS / NCOPY;
    bf16x8 kf[3];
    float lsa = 0.0f, lsb = 0.0f;  // row sum of the stage's probabilities (fp32)
    kf[0] = *reinterpret_cast<const bf16x8*>(kb + koffs[0]);
    kf[1] = *reinterpret_cast<const bf16x8*>(kb + koffs[1]);
#pragma unroll
    for (int r = 0; r < 16; ++r) s_nxt[r] = 0.0f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      if (k + 2 < KS) kf[(k + 2) % 3] = *reinterpret_cast<const bf16x8*>(kb + koffs[k + 2]);
      s_nxt = mfma(kf[k % 3], qf[k], s_nxt);
      // The copy instructions spread evenly over the slots (V of u + R - 1,
      // then K of u + R).
      if (k % CEVERY == 0) {
        const int c = k / CEVERY;
        if (c < NL) {
          copy_v_at(std::integral_constant<int, VNEW>{}, c, srow[R - 2]);
        } else {
          copy_k_at(std::integral_constant<int, KNEW>{}, c - NL, srow[R - 1]);
        }
      }
#pragma unroll
      for (int x = 0; x < EXP_PER; x += 2) {
        const int r = k * EXP_PER + x;
        float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r], sl2, -m_use));
        float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[r + 1], sl2, -m_use));
        // Pin the exponentials to this slot: without it the compiler sinks
        // the softmax below the masking branch, after every QK^T MFMA.
        asm volatile("" : "+v"(e0), "+v"(e1));
        pf[r / 8][r % 8] = (__bf16)e0;
        pf[r / 8][r % 8 + 1] = (__bf16)e1;
        lsa += e0;
        lsb += e1;
      }
#pragma unroll
      for (int x = 0; x < VRD_PER; ++x) {
        const int idx = k * VRD_PER + x;
        const int dt = idx / 2, c2 = idx % 2;
        vf0[dt][c2] = vread(VB, 0, dt, c2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lsum += lsa + lsb;

    // With no stage u + 1 (past the end of the list) S[u+1] is a product of
    // K data already in LDS with every key masked: the softmax state stays.
    mask(s_nxt, u + 1 < nst ? snv[0] : 0, srow[0]);
    // ---- (b) O += V^T P[u]^T || row max of S[u+1].
    float mxl = -__builtin_inff();
    constexpr int NPV = 2 * DT;
#pragma unroll
    for (int sl = 0; sl < NPV; ++sl) {
      const int ks2 = sl / DT, dt = sl % DT;
      if (sl < DT) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) vf1[sl][c2] = vread(VB, 1, sl, c2);
      }
      const bf16x4* vf = ks2 == 0 ? vf0[dt] : vf1[dt];
      const bf16x8 av = __builtin_shufflevector(vf[0], vf[1], 0, 1, 2, 3, 4, 5, 6, 7);
      o[dt] = mfma(av, pf[ks2], o[dt]);
#pragma unroll
      for (int it = sl * 8 / NPV; it < (sl + 1) * 8 / NPV; ++it) {
        mxl = __builtin_fmaxf(mxl, __builtin_fmaxf(s_nxt[2 * it], s_nxt[2 * it + 1]));
        asm volatile("" : "+v"(mxl));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    check_ref(mxl);
    cur_nv = snv[0];
  };

  // R steps per loop turn so that the LDS stages and the S registers are
  // compile-time indices. The last stage runs the same step: its S[u+1] is
  // a product of K data already in LDS with every key masked, which leaves
  // the softmax state unchanged (a separate last step would need registers
  // the loop does not have); its copies read the last stage's rows again.
  for (int u = 0; u < nst; u += R) {
    run_step(std::integral_constant<int, 0>{}, u);
    if (u + 1 >= nst) break;
    run_step(std::integral_constant<int, 1>{}, u + 1);
    if constexpr (R == 4) {
      if (u + 2 >= nst) break;
      run_step(std::integral_constant<int, 2 % R>{}, u + 2);
      if (u + 3 >= nst) break;
      run_step(std::integral_constant<int, 3 % R>{}, u + 3);
    }
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

// LDS of a workgroup: R K stages and R V stages, or the epilogue's
// hand-over area if that is larger.
template <int D, int NQG>
constexpr int smem_elems() {
  constexpr int stages = 2 * kv_ring<D, NQG>() * 64 * D;
  constexpr int handover = 2 * NQG * ((D / 64) * 16 + 2) * 64 * 2;  // floats -> bf16 units
  return stages > handover ? stages : handover;
}

// Waves per SIMD: two at head_dim 128 (up to 256 VGPRs each), three at
// head_dim 64 (up to 168).
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
  AttnParams q = p;
  q.even_share16 = pair_split<D, NQG>(p);
  const int pj0 = (p.n_wg >> 2) + ((p.n_wg & 3) ? 1 : 0);  // the largest pair's work
  const int tot = p.nq * p.group * p.qparts;                 // per (batch, KV head)
  const int per_head = q.even_share16 == 32768 ? (tot + 7) / 8
                                               : even_count((tot >> 2) + ((tot & 3) ? 1 : 0),
                                                            q.even_share16);
  const int grid = p.head_sync ? p.batch * p.hkv * 8 * per_head
                               : 8 * even_count(pj0, q.even_share16);
  hipLaunchKernelGGL((attn_fwd_kernel<D, BK, NQG, MODE>), dim3(grid), dim3(128 * NQG), 0, stream,
                     q);
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
