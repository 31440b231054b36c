// Selected-block attention forward kernel for gfx950 (CDNA4).
//
// What it computes (vllm-omni PR #8335 "[Core] Add shared block-sparse
// attention adapters with FlashAttention-4", Purpose; diffusers
// examples/cosmos3/cosmos_parallel.py, cosmos3_cp_attention and
// build_gen_key_mask): for every query row of a query block, non-causal
// softmax attention over the keys of the KV blocks listed for that
// (batch, query head, query block), padded keys excluded, query head h
// reading KV head h / G in place. The dense case is the same kernel with the
// list "every non-empty block" generated in-kernel.
//
// Structure (one workgroup per query block, one wave per 32 query rows):
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the K tile (A operand) comes
//    from LDS, Q^T (B operand) stays in registers for the whole row block.
//    Each lane then owns one query row (lane % 32) and half of the tile's
//    keys, so the row max / row sum need a single cross-lane step.
//  * Online softmax in fp32, exp2 with the scale folded into one FMA.
//  * O^T = V^T P^T with the same MFMA: P^T is the S^T accumulator converted
//    to bf16 in place (the contraction over keys is order-free, so the key
//    order of the accumulator layout is reused for V); V^T fragments are
//    read from the row-major V tile with ds_read_b64_tr_b16. The output
//    accumulator again has one query per lane, so the softmax rescale is a
//    per-lane multiply.
//  * K and V tiles move HBM -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging), XOR-swizzled in 16-byte chunks so the K row reads and the
//    V transpose reads hit distinct banks. K of the next block loads while
//    this block's softmax and PV run; V of the next block loads while the
//    next QK^T and softmax run.
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
// keeps the K reads conflict-free.
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

// HBM->LDS copy of one [BK x D] bf16 tile with global_load_lds_dwordx4 in its
// scalar-base form: the LDS destination comes from M0 and the HBM address is
// a 64-bit scalar base plus a 32-bit per-lane offset, so issuing a copy costs
// no vector ALU work. Each wave instruction moves 64 x 16 bytes = RPI whole
// rows; instruction `it` of wave `wave` fills rows (it * NW + wave) * RPI +
// [0, RPI). The row step between instructions is a multiple of 8 rows, so the
// XOR swizzle of a lane's chunk is the same for every instruction and the
// per-lane offset is fixed for the whole kernel.
//
// The copies are issued from inline assembly, so the compiler does not track
// them: every read of a tile is preceded by an explicit wait_vmcnt on the
// copies that must have landed and an LDS barrier.
template <int D, int BK, int NW>
struct TileCopy {
  static constexpr int CPR = D / 8;
  static constexpr int RPI = 64 / CPR;
  static constexpr int NL = BK / (NW * RPI);
  static_assert(NL * NW * RPI == BK, "tile split");
  uint32_t voff[NL];  // per-lane byte offset of instruction `it` inside the tile
  uint32_t lds_base;  // uniform LDS byte address of this wave's first rows

  __device__ __forceinline__ void init(int64_t row_stride, int wave, int lane, const uint16_t* lds) {
#pragma unroll
    for (int it = 0; it < NL; ++it) {
      const int row = (it * NW + wave) * RPI + lane / CPR;
      const int lch = (lane % CPR) ^ swz<CPR>(row);
      voff[it] = (uint32_t)((row * row_stride + lch * 8) * 2);
    }
    lds_base = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint16_t*)lds) +
               (uint32_t)(wave * RPI * D * 2);
  }
  template <int IT>
  __device__ __forceinline__ void one(const uint16_t* tile, uint32_t lbase) const {
    asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff[IT]), "s"(tile), "s"(lbase), "i"(IT * NW * RPI * D * 2)
                 : "memory", "m0");
  }
  template <int... IT>
  __device__ __forceinline__ void all(const uint16_t* tile, uint32_t lbase,
                                      std::integer_sequence<int, IT...>) const {
    (one<IT>(tile, lbase), ...);
  }
  // `tile` is the uniform address of row 0 of the tile; `lds_off` selects
  // the LDS buffer (bytes). Each copy instruction costs one scalar add (its
  // LDS destination) besides the copy itself.
  __device__ __forceinline__ void issue(const uint16_t* tile, uint32_t lds_off = 0) const {
    all(tile, lds_base + lds_off, std::make_integer_sequence<int, NL>{});
  }
};

// Uniform 32-bit load through the scalar data cache (the index list is
// read-only here); waits for its own completion.
__device__ __forceinline__ int scalar_load_i32(const int32_t* ptr) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
  return v;
}

// Value of the other half-wave: lanes l and l ^ 32 hold the same query row.
__device__ __forceinline__ float max_with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Kernel body. One wave per 32 query rows; the keys of each listed KV block
// are processed as sub-tiles of 64 keys. K and V tiles are double-buffered in
// LDS and each step starts with the only workgroup barrier of the step: the
// copies issued one step earlier have landed and the buffers read in the
// previous step are free for the next copies. Per sub-tile u a wave then runs
//   (a) S[u+1] = K Q^T on the matrix cores, interleaved instruction by
//       instruction with the exponentials of P[u] (the row maxima of S[u]
//       are already known) and the V transpose reads for step (b);
//   (b) O += V^T P[u]^T and the row sums of P[u] on the matrix cores,
//       interleaved with the masking and row maxima of S[u+1].
// One wave per SIMD: the matrix cores and the vector ALUs are kept busy by
// the interleaving inside the wave rather than by switching waves.
template <int D, int BQ, int BK, bool DENSE>
__device__ __forceinline__ void attn_fwd_body(const AttnParams& p, uint16_t* __restrict__ Ks,
                                              uint16_t* __restrict__ Vs) {
  constexpr int NW = BQ / 32;
  constexpr int CPR = D / 8;
  constexpr int KS = D / 16;    // MFMA k-steps over D
  constexpr int DT = D / 32;    // output 32-row tiles over D
  constexpr int SUB = 64;       // keys per pipeline sub-tile
  constexpr int KT = SUB / 32;  // 32-key MFMA tiles per sub-tile
  constexpr int SPB = BK / SUB; // sub-tiles per KV block
  constexpr int NQK = KS * KT;  // QK^T MFMAs per sub-tile
  constexpr int TILE = BK * D;  // elements of one K or V buffer
  static_assert(NQK == 16 || NQK == 8, "interleave assumes 8 or 16 QK^T MFMAs");
  using Copy = TileCopy<D, BK, NW>;
  // A row moves its reference max only when a sub-tile max exceeds it by
  // more than this many powers of two; until then probabilities are taken
  // against the stale max and stay below 2^8, far from fp32 or bf16 overflow.
  constexpr float kRescaleSlack = 8.0f;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;

  // Workgroup w runs on XCD w % 8; give each XCD a contiguous range of the
  // (batch, KV head, query block, head-in-group) order.
  const int nwg = p.n_wg;
  const int w = blockIdx.x;
  const int xcd = w & 7, per = nwg >> 3, rem = nwg & 7;
  const int lin = xcd * per + min(xcd, rem) + (w >> 3);
  const int hig = lin % p.group;
  int t = lin / p.group;
  const int i = t % p.nq;
  t /= p.nq;
  const int g = t % p.hkv;
  const int b = t / p.hkv;
  const int h = g * p.group + hig;

  const int row0 = i * BQ;
  const int qrow = row0 + wave * 32 + col;

  // Q^T fragments (B operand): lane holds q[qrow][16 ks + 8 half .. +7].
  bf16x8 qf[KS];
  {
    const uint16_t* qp = p.q + (int64_t)b * p.qs0 + (int64_t)qrow * p.qs1 + (int64_t)h * p.qs2 +
                         half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
    // Retire these loads now: the tile copies below are counted on the same
    // vector-memory counter and are awaited explicitly.
    wait_vmcnt<0>();
  }

  int nblk;
  const int32_t* idx_row = nullptr;
  if constexpr (DENSE) {
    nblk = p.n_forced + p.n_cand;
  } else {
    const int64_t row_id = ((int64_t)b * p.hq + h) * p.nq + i;
    nblk = min(max(scalar_load_i32(p.cnt + row_id), 0), p.idx_row_stride);
    idx_row = p.idx + row_id * p.idx_row_stride;
  }
  if (row0 >= p.q_valid || p.nk == 0) nblk = 0;

  const uint16_t* kbase = p.k + (int64_t)b * p.ks0 + (int64_t)g * p.ks2;
  const uint16_t* vbase = p.v + (int64_t)b * p.vs0 + (int64_t)g * p.vs2;
  Copy kcopy, vcopy;
  kcopy.init(p.ks1, wave, lane, Ks);
  vcopy.init(p.vs1, wave, lane, Vs);

  // Listed block n. Entries outside [0, NK) are copied from block 0 (always
  // in bounds) with no real key, which gives them zero weight.
  auto block_of = [&](int n) -> int {
    if constexpr (DENSE) {
      return n < p.n_forced ? n : p.n_prefix_blocks + (n - p.n_forced);
    } else {
      return scalar_load_i32(idx_row + n);
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
  auto load_of = [&](int j) -> int64_t { return (j < 0 || j >= p.nk) ? 0 : (int64_t)j * BK; };

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.0f;
  // Row sums of P come out of the matrix core: ones(32 x 16) x P^T puts the
  // sum over a 16-key step into every row of the accumulator (one query per
  // lane); entry 0 is the one kept.
  f32x16 lacc;
#pragma unroll
  for (int r = 0; r < 16; ++r) lacc[r] = 0.0f;
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  const float sl2 = p.scale_log2;

  // LDS element offsets that do not depend on the block.
  const int sw = swz<CPR>(col);  // swizzle of K rows 32 kt + col
  int koffs[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koffs[ks] = col * D + (((2 * ks + half) ^ sw) << 3);
  const int g16 = lane >> 4, j16 = lane & 15, tq = j16 >> 2, q4 = j16 & 3;
  int voffs[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int d = dt * 32 + 16 * (g16 & 1) + 4 * q4;
      const int row = 8 * c2 + 4 * half + tq;  // + multiples of 16
      voffs[dt][c2] = row * D + (((d >> 3) ^ swz<CPR>(row)) << 3) + (d & 7);
    }

  // Softmax state of the sub-tile about to be finished.
  float m_run = -__builtin_inff();  // reference max (log2 units) of this row
  float m_use = 0.0f, alpha = 1.0f;
  bool need = false;
  // Mask, row max and reference update for a freshly computed S (keys of the
  // sub-tile at or past `nvs` are padding).
  auto mask = [&](f32x16 (&sd)[KT], int nvs) {
    if (nvs < SUB) {  // only sub-tiles that hold padding (uniform branch)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
          sd[kt][r] = key < nvs ? sd[kt][r] : -__builtin_inff();
        }
    }
  };
  auto prep = [&](f32x16 (&sd)[KT]) {
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        mx = __builtin_fmaxf(mx, __builtin_fmaxf(sd[kt][r], sd[kt][r + 1]));
    mx = max_with_other_half(mx) * sl2;
    need = mx > m_run + kRescaleSlack;
    const float e_alpha = __builtin_amdgcn_exp2f(m_run - mx);
    alpha = need ? e_alpha : 1.0f;
    m_run = need ? mx : m_run;
    m_use = (m_run == -__builtin_inff()) ? 0.0f : m_run;
  };

  // Block bookkeeping: nv0 = real keys of block n; (j1, nv1) block n+1;
  // (j2, nv2) block n+2.
  int nv0 = 0, j1 = -1, nv1 = 0, j2 = -1, nv2 = 0;
  f32x16 sA[KT], sB[KT];

  if (nblk > 0) {
    const int j0 = block_of(0);
    nv0 = nvalid_of(j0);
    kcopy.issue(kbase + load_of(j0) * p.ks1, 0);
    vcopy.issue(vbase + load_of(j0) * p.vs1, 0);
    if (nblk > 1) {
      j1 = block_of(1);
      nv1 = nvalid_of(j1);
      kcopy.issue(kbase + load_of(j1) * p.ks1, TILE * 2);
    }
    wait_vmcnt<0>();
    lds_barrier();
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sA[kt][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + kt * 32 * D + koffs[ks]);
        sA[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sA[kt], 0, 0, 0);
      }
    mask(sA, nv0);
    prep(sA);
  }

  // One pipeline step on sub-tile `sub` of block n. KP / VP are the LDS
  // buffers read in this step (K of the next sub-tile, V of this one).
  auto step = [&](auto kp_c, auto vp_c, int n, int sub, f32x16 (&s_cur)[KT],
                  f32x16 (&s_nxt)[KT]) {
    constexpr int KP = decltype(kp_c)::value;
    constexpr int VP = decltype(vp_c)::value;
    const bool last_sub = sub == SPB - 1;
    const bool has_next = !last_sub || n + 1 < nblk;
    if (last_sub) {
      j2 = (n + 2 < nblk) ? block_of(n + 2) : -1;
      nv2 = (n + 2 < nblk) ? nvalid_of(j2) : 0;
    }
    // ---- the step's single synchronisation point.
    wait_vmcnt<0>();
    lds_barrier();
    if (sub == 0 && n + 1 < nblk) vcopy.issue(vbase + load_of(j1) * p.vs1, (VP ^ 1) * TILE * 2);
    if (last_sub && n + 2 < nblk) kcopy.issue(kbase + load_of(j2) * p.ks1, (KP ^ 1) * TILE * 2);
    const uint16_t* kb = Ks + KP * TILE + (last_sub ? 0 : (sub + 1) * SUB * D);
    const uint16_t* vb = Vs + VP * TILE + sub * SUB * D;
    if (sub == 0 && nv0 < BK) {
      // Padded keys get weight 0, but 0 * NaN is NaN: clear their V rows.
      constexpr int NT = NW * 64;
      uint4* vz = reinterpret_cast<uint4*>(Vs + VP * TILE + nv0 * D);
      const int nz = (BK - nv0) * D / 8;
      for (int e = threadIdx.x; e < nz; e += NT) vz[e] = make_uint4(0, 0, 0, 0);
      lds_barrier();
    }
    // Lazy rescale of the running output (rare after the first sub-tiles).
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      lacc[0] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }

    // ---- (a) S[u+1] = K Q^T || exponentials of P[u] || V^T reads.
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s_nxt[kt][r] = 0.0f;
    bf16x8 pf[2 * KT];
    bf16x4 vf[2 * KT][DT][2];
    constexpr int EXP_PER = (2 * KT * 8) / NQK;   // exponentials per MFMA slot
    constexpr int VRD_PER = (2 * KT * DT * 2) / NQK;  // V reads per MFMA slot
    // K fragments are read two MFMA slots ahead of their use.
    constexpr int KPF = 2;
    bf16x8 kf[KPF + 1];
#pragma unroll
    for (int k = 0; k < KPF; ++k)
      kf[k] = *reinterpret_cast<const bf16x8*>(kb + (k % KT) * 32 * D + koffs[k / KT]);
#pragma unroll
    for (int k = 0; k < NQK; ++k) {
      const int ks = k / KT, kt = k % KT;
      if (k + KPF < NQK)
        kf[(k + KPF) % (KPF + 1)] = *reinterpret_cast<const bf16x8*>(
            kb + ((k + KPF) % KT) * 32 * D + koffs[(k + KPF) / KT]);
      s_nxt[kt] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k % (KPF + 1)], qf[ks], s_nxt[kt], 0, 0, 0);
#pragma unroll
      for (int x = 0; x < EXP_PER; ++x) {
        const int idx = k * EXP_PER + x;           // element of P[u], 0 .. 16 KT - 1
        const int pk = idx / 8, pe = idx % 8;      // fragment and slot
        const int skt = pk / 2, sr = 8 * (pk % 2) + pe;
        pf[pk][pe] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[skt][sr], sl2, -m_use));
      }
#pragma unroll
      for (int x = 0; x < VRD_PER; ++x) {
        const int idx = k * VRD_PER + x;           // 0 .. 4 KT DT - 1
        const int ks2 = idx / (DT * 2), dt = (idx / 2) % DT, c2 = idx % 2;
        const int kt2 = ks2 / 2, s2 = ks2 % 2;
        vf[ks2][dt][c2] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(vb + (kt2 * 32 + 16 * s2) * D + voffs[dt][c2]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // With no next sub-tile, S[u+1] is a dummy product and every key of it
    // counts as padding, which leaves the softmax state unchanged.
    const int nvs_next = !has_next ? 0 : (last_sub ? nv1 : nv0 - (sub + 1) * SUB);
    mask(s_nxt, nvs_next);
    // ---- (b) O += V^T P[u]^T and row sums || row max of S[u+1].
#pragma unroll
    for (int ks2 = 0; ks2 < 2 * KT; ++ks2) {
      lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pf[ks2], lacc, 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 av =
            __builtin_shufflevector(vf[ks2][dt][0], vf[ks2][dt][1], 0, 1, 2, 3, 4, 5, 6, 7);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf[ks2], o[dt], 0, 0, 0);
      }
    }
    prep(s_nxt);

    if (last_sub) {
      nv0 = nv1;
      j1 = j2;
      nv1 = nv2;
    }
  };

  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  // Steps in order, two blocks per loop turn so that the LDS buffers and the
  // S registers alternate statically.
  for (int n = 0; n < nblk; n += 2) {
    if constexpr (SPB == 1) {
      step(C1{}, C0{}, n, 0, sA, sB);
      if (n + 1 < nblk) step(C0{}, C1{}, n + 1, 0, sB, sA);
    } else {
      step(C0{}, C0{}, n, 0, sA, sB);
      step(C1{}, C0{}, n, 1, sB, sA);
      if (n + 1 < nblk) {
        step(C1{}, C1{}, n + 1, 0, sA, sB);
        step(C0{}, C1{}, n + 1, 1, sB, sA);
      }
    }
  }

  // ---- epilogue: O^T lane layout is query col, d = dt*32 + (r/4)*8 + half*4 + r%4.
  const float l_run = lacc[0];
  const bool row_ok = qrow < p.q_valid && l_run > 0.0f;
  const float inv = row_ok ? 1.0f / l_run : 0.0f;
  uint16_t* op = p.o + (int64_t)b * p.os0 + (int64_t)qrow * p.os1 + (int64_t)h * p.os2;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      bf16x4 vv;
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[e] = (__bf16)(row_ok ? o[dt][rg * 4 + e] * inv : 0.0f);
      *reinterpret_cast<bf16x4*>(op + dt * 32 + rg * 8 + half * 4) = vv;
    }
  if (p.lse != nullptr && half == 0) {
    const float lse = row_ok ? (m_run + __builtin_log2f(l_run)) * 0.69314718055994531f
                             : -__builtin_inff();
    p.lse[((int64_t)b * p.hq + h) * p.q_len + qrow] = lse;
  }
}

template <int D, int BQ, int BK, bool DENSE>
__global__ void __launch_bounds__(BQ * 2) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_fwd_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2 * BK * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2 * BK * D];
  attn_fwd_body<D, BQ, BK, DENSE>(p, Ks, Vs);
}

template <int D, int BQ, int BK, bool DENSE>
hipError_t launch_one(const AttnParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, BQ, BK, DENSE>), dim3(p.n_wg), dim3(BQ * 2), 0, stream,
                     p);
  return hipGetLastError();
}

template <int D, int BQ, int BK>
hipError_t launch_mode(const AttnParams& p, bool dense, hipStream_t stream) {
  return dense ? launch_one<D, BQ, BK, true>(p, stream) : launch_one<D, BQ, BK, false>(p, stream);
}

template <int D>
hipError_t launch_geom(const AttnParams& p, int bq, int bk, bool dense, hipStream_t stream) {
  if (bq == 64 && bk == 64) return launch_mode<D, 64, 64>(p, dense, stream);
  if (bq == 64 && bk == 128) return launch_mode<D, 64, 128>(p, dense, stream);
  if (bq == 128 && bk == 64) return launch_mode<D, 128, 64>(p, dense, stream);
  return launch_mode<D, 128, 128>(p, dense, stream);
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, int head_dim, int block_q, int block_k, bool dense,
                            hipStream_t stream) {
  if (p.n_wg == 0) return hipSuccess;
  if (head_dim == 128) return launch_geom<128>(p, block_q, block_k, dense, stream);
  return launch_geom<64>(p, block_q, block_k, dense, stream);
}

}  // namespace bsattn
