// Internal declarations shared by the host entry points and the kernels of
// libbsattn. Not part of the public ABI (that is include/bsattn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsattn.h"

namespace bsattn {

// Kernel-side description of one attention call (all sizes validated on the
// host before any launch).
struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;            // may be null
  const int32_t* idx;    // sparse only
  const int32_t* cnt;    // sparse only
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;
  int32_t batch, hq, hkv, group;
  int32_t q_len, q_valid, kv_prefix_len, kv_prefix_valid, kv_suffix_valid;
  int32_t nq, nk;
  int32_t n_prefix_blocks;  // P
  int32_t n_forced;         // protected blocks holding a real key: [0, n_forced)
  int32_t n_cand;           // generation blocks holding a real key: [P, P + n_cand)
  int32_t idx_row_stride;
  int32_t causal_off;       // causal mode: real keys - real query rows (bottom-right alignment)
  int32_t qparts;           // workgroups per query block: block_q / 128 above 128 rows, else 1
  int32_t n_wg;             // workgroups with work: batch * hq * nq * qparts
  int32_t head_sync;        // 1: all XCDs on one KV head at a time (grid padded per head)
  int32_t even_share16;     // 65536 x the share of each XCD pair's work its even XCD takes
  float scale_log2;         // softmax scale * log2(e)
  // Bytes from the first K (V) element of a (batch, KV head) to one past its
  // last one: the range of the copies' buffer resource (below 2^31).
  uint32_t k_span_bytes, v_span_bytes;
};

struct PoolParams {
  const uint16_t* q;
  const uint16_t* k;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2;
  int32_t hq, hkv, bq, bk, q_valid, kv_prefix_len, kv_prefix_valid, kv_suffix_valid;
  int32_t nq, nk;
  double* qp;    // [B][Hq][NQ][D]  pooled queries (fp32 values held exactly in fp64)
  double* qn;    // [B][Hq][NQ]     upper bound of the L2 norm of each pooled query
  float* kpt;    // [B][Hkv][D][NK] pooled keys, transposed
  double* kn;    // [B][Hkv][NK]    upper bound of the L2 norm of each pooled key
};

struct ScoreParams {
  const double* qp;
  const double* qn;
  const float* kpt;
  const double* kn;
  int32_t* idx;
  int32_t* cnt;
  int32_t hq, hkv, group, nq, nk, bq, q_valid;
  int32_t n_prefix_blocks, n_forced, n_cand, keep, idx_row_stride;
};

// Attention modes: the listed blocks, every non-empty block, or every block
// up to the causal limit with the diagonal masked.
enum AttnMode : int { kSparse = 0, kDense = 1, kCausal = 2 };

// Launchers (return the HIP error of the launch).
hipError_t launch_attention(const AttnParams& p, int head_dim, int block_q, int block_k, int mode,
                            hipStream_t stream);
hipError_t launch_pool(const PoolParams& p, int head_dim, int batch, hipStream_t stream);
hipError_t launch_score_topk(const ScoreParams& p, int head_dim, int batch, hipStream_t stream);

// Records a failure of entry point `fn` for attn_last_error() (the message
// gains the library version and target) and returns `st`; ATTN_OK clears
// the record.
attn_status report(attn_status st, const char* fn, const char* msg);

// Rows of the score kernel per workgroup and its dynamic LDS bytes.
int score_rows_per_wg(int n_cand);
size_t score_lds_bytes(int n_cand);

}  // namespace bsattn
