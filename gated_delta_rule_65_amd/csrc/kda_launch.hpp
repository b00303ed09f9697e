// Host-side launch descriptors between the C-ABI layer and the kernel files.
#pragma once
#include "kda_common.hpp"
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct DecodeLaunch {
  const void *q, *k, *v, *g, *beta;
  void* cache;                // fp32 or bf16 (state_bf16)
  int state_bf16;
  const int32_t* idx;
  void* out;
  int dtype, n, hqk, hv, use_l2, num_slots;
  float scale;
  void* stream;
  GateArgs gate;  // optional gate parameters (a_log == NULL: none)
  int tokens;                 // tokens per request (1..8)
  int cols;                   // columns of a 2-D state_indices, 0 for 1-D
  const int32_t* accepted;    // [n] accepted-token counts or NULL
  InStrides strides;          // per-token input strides (resolved, never 0)
  int64_t slot_stride;        // elements between cache slots (resolved)
};
hipError_t launch_decode(const DecodeLaunch& L);

// The record-based verify window (outputs and records, no state).
struct VerifyLaunch {
  const void *q, *k, *v, *g, *beta;
  const int32_t* query_start;  // [n + 1]
  const void* cache;           // fp32 or bf16 (state_bf16), read only
  int state_bf16;
  const int32_t* idx;          // [n] slots
  float* corr;                 // [n, hv, window, 128]
  void* kg;                    // [n, hv, window, 256], input dtype
  void* out;                   // [T, hv, 128]
  int dtype, n, hqk, hv, window, use_l2, num_slots;
  float scale;
  GateArgs gate;
  InStrides strides;
  int64_t slot_stride;
  void* stream;
};
hipError_t launch_verify(const VerifyLaunch& L);

// The commit of the accepted prefix from the verify records.
struct CommitLaunch {
  void* cache;
  int state_bf16;
  const int32_t* idx;          // [n] slots
  const int32_t* accepted;     // [n]
  const float* corr;
  const void* kg;
  int dtype, n, hv, window, use_l2, num_slots;
  GateArgs gate;
  int64_t slot_stride;
  void* stream;
};
hipError_t launch_commit(const CommitLaunch& L);

// The staged chunked forward: every buffer already carved from the workspace.
struct ChunkLaunch {
  const void *q, *k, *v, *g, *beta;
  const int32_t* cu;          // [N+1] (device) or NULL for dense
  int dtype, num_seqs, hqk, hv, use_l2;
  int64_t total_tokens, max_chunks;
  float scale;
  const void* init;           // dense initial state or NULL (fp32, or bf16 with state_bf16)
  void* fin;                  // dense final state or NULL (same storage)
  int state_bf16;
  void* cache;                // paged state (fp32, or bf16 with state_bf16) or NULL
  const int32_t* slots;
  const uint8_t* has_init;
  int num_slots;
  void* out;
  // workspace pieces
  int32_t* chunk_offsets;     // [N+1]
  void* table;                // int4 [max_chunks]: (sequence, first token, length, 0)
  void *qg, *kg_t, *w, *u, *aqk;
  float* decay;
  float* scan;                // group-scan planes (groups > 1)
  void* zero;                 // 1 KiB zero page (written by the chunk-table kernel)
  int groups;                 // chunk groups per sequence (1 = plain walk)
  int walk_waves;             // waves per walk workgroup: 2, 4 or 8 (16 columns each)
  int fuse_prep;              // 1: the WY kernel also writes qg, kg_t and decay
  GateArgs gate;  // optional gate parameters (a_log == NULL: none)
  float* ckpt;                // state snapshots [rows, Hv, 128, 128] or NULL
  const int32_t* ckpt_off;    // [N] token offsets
  const int32_t* ckpt_idx;    // [N] destination rows or NULL (row n)
  int ckpt_rows;
  InStrides strides;          // per-token input strides (resolved, never 0)
  int64_t slot_stride;        // elements between paged state slots (resolved)
  void** events;              // optional stage events (KDA_EV_*), may be NULL
  int num_events;
  void* stream;
};
hipError_t launch_chunk_staged(const ChunkLaunch& L);
// The on-chip path (bf16): the intra-chunk stage inside the walk; the
// workspace holds only the chunk table and the group-scan planes.
hipError_t launch_chunk_onchip(const ChunkLaunch& L);
// The chunk-table kernel alone (offsets, records, zero page).
void launch_chunk_table(const ChunkLaunch& L);
// Compute units of the current device (256 when the query fails).
int cu_count_host();

}  // namespace kda
