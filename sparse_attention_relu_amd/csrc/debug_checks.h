// Precondition rules of the C ABI that depend on device data, written once
// for both sides: the SA_DEBUG build's check kernels call them on the device,
// sa_debug_check_host calls them on host arrays.  Each returns 0 when the item
// is valid, else an SA_DBG_* code and the offending value in *val.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sparse_mla.h"

namespace sa_dbg {

enum Code : uint32_t {
  OK = 0,
  Q_SEQ_RANGE = 1,        // q_seq[t] outside [0, n_seq)
  Q_POS_NEG = 2,          // q_pos[t] < 0
  Q_POS_BEYOND_SEQ = 3,   // q_pos[t] >= seq_len[q_seq[t]]
  Q_POS_BEYOND_LD = 4,    // q_pos[t] >= ld
  SEQ_LEN_RANGE = 5,      // seq_len[b] outside [0, SA_MAX_SEQ_LEN]
  SEQ_START_NEG = 6,      // seq_start[b] < 0
  IDX_RANGE = 7,          // idx[t, j] < -1, >= SA_MAX_SEQ_LEN, or (when known) > q_pos[t]
  SCORE_NAN = 8,          // a NaN among scores[t, 0 .. q_pos[t]]
  CACHE_POS_NEG = 9,      // cache write: pos[i] < 0
  CACHE_DST_NEG = 10,     // cache write: dst[i] < 0
  SEL_OF_RANGE = 11,      // shared selection: sel_of[t] outside [0, n_sel)
  SEL_SEQ_MISMATCH = 12,  // shared selection: sel_seq[sel_of[t]] != q_seq[t]
  N_CODES = 13
};

// Record layout (device word array and host report alike):
// [0] first code, [1] its item (query, sequence or token), [2] its slot
// (selection slot, or 0), [3] low 32 bits of the offending value, [4] number
// of violations seen.
constexpr int kRecWords = 8;

__host__ __device__ inline const char* code_name(uint32_t c) {
  switch (c) {
    case Q_SEQ_RANGE: return "q_seq outside [0, n_seq)";
    case Q_POS_NEG: return "q_pos negative";
    case Q_POS_BEYOND_SEQ: return "q_pos not below its sequence's seq_len";
    case Q_POS_BEYOND_LD: return "q_pos not below ld";
    case SEQ_LEN_RANGE: return "seq_len outside [0, SA_MAX_SEQ_LEN]";
    case SEQ_START_NEG: return "seq_start negative";
    case IDX_RANGE: return "idx entry outside [-1, q_pos] (or beyond SA_MAX_SEQ_LEN)";
    case SCORE_NAN: return "NaN score in a row the top-k reads";
    case CACHE_POS_NEG: return "cache-write position negative";
    case CACHE_DST_NEG: return "cache-write row negative";
    case SEL_OF_RANGE: return "sel_of outside [0, n_sel)";
    case SEL_SEQ_MISMATCH: return "selecting query of another sequence";
    default: return "unknown check";
  }
}

// Query t of a batch.  seq_len may be null (the attention call has none),
// n_seq < 0 means unknown, ld < 0 means unknown.
__host__ __device__ inline uint32_t check_query(int32_t q_seq, int32_t q_pos, const int32_t* seq_len, int32_t n_seq,
                                                int64_t ld, int64_t* val) {
  if (q_seq < 0 || (n_seq >= 0 && q_seq >= n_seq)) {
    *val = q_seq;
    return Q_SEQ_RANGE;
  }
  if (q_pos < 0) {
    *val = q_pos;
    return Q_POS_NEG;
  }
  if (seq_len && q_pos >= seq_len[q_seq]) {
    *val = q_pos;
    return Q_POS_BEYOND_SEQ;
  }
  if (ld >= 0 && (int64_t)q_pos >= ld) {
    *val = q_pos;
    return Q_POS_BEYOND_LD;
  }
  return OK;
}

// Sequence b of a batch.
__host__ __device__ inline uint32_t check_sequence(int64_t seq_start, int32_t seq_len, int64_t* val) {
  if (seq_len < 0 || seq_len > SA_MAX_SEQ_LEN) {
    *val = seq_len;
    return SEQ_LEN_RANGE;
  }
  if (seq_start < 0) {
    *val = seq_start;
    return SEQ_START_NEG;
  }
  return OK;
}

// One selection entry; q_pos < 0 means the causal bound is unknown.
__host__ __device__ inline uint32_t check_idx(int32_t idx, int32_t q_pos, int64_t* val) {
  if (idx < -1 || idx >= SA_MAX_SEQ_LEN || (q_pos >= 0 && idx > q_pos)) {
    *val = idx;
    return IDX_RANGE;
  }
  return OK;
}

// Query t of a batch with a shared selection; sel_seq may be null (the
// sequences are unknown: only the range of sel_of is checked).
__host__ __device__ inline uint32_t check_share(int32_t sel_of, int32_t n_sel, int32_t q_seq, const int32_t* sel_seq,
                                                int64_t* val) {
  if (sel_of < 0 || sel_of >= n_sel) {
    *val = sel_of;
    return SEL_OF_RANGE;
  }
  if (sel_seq && sel_seq[sel_of] != q_seq) {
    *val = sel_seq[sel_of];
    return SEL_SEQ_MISMATCH;
  }
  return OK;
}

}  // namespace sa_dbg
