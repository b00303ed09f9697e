// C-ABI entry points of the KDA library: argument checks, workspace carving,
// launch plans.  Every check runs on the host before anything is queued; a
// failed check returns a status and writes nothing.
#include <math.h>

#include <cmath>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "../../include/kda.h"
#include "kda_launch.hpp"

#define KDA_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

kda_status fail(kda_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

kda_status ok() {
  g_err[0] = '\0';
  return KDA_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t elem_size(int dtype) { return dtype == KDA_F32 ? 4 : 2; }

// Tensor base pointers are read with 8- and 16-byte vector loads.
bool misaligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (reinterpret_cast<uintptr_t>(p) & 15) return true;
  return false;
}

// Resolves the optional per-token input strides (0 = dense) and checks them:
// at least the dense stride, at most 2^24 elements, and 16-byte token rows
// for the vector-loaded inputs.
kda_status resolve_strides(int64_t q, int64_t k, int64_t v, int64_t g, int64_t b, int hqk,
                           int hv, size_t es, kda::InStrides& out) {
  const int64_t dq = (int64_t)hqk * KDA_HEAD_DIM, dv = (int64_t)hv * KDA_HEAD_DIM;
  const int64_t in[5] = {q, k, v, g, b}, dense[5] = {dq, dq, dv, dv, hv};
  const char* names[5] = {"q", "k", "v", "g", "beta"};
  int64_t r[5];
  for (int i = 0; i < 5; ++i) {
    r[i] = in[i] ? in[i] : dense[i];
    if (r[i] < dense[i] || r[i] > ((int64_t)1 << 24))
      return fail(KDA_ERR_SHAPE, "%s_stride %lld must be 0 or in [%lld, 2^24]", names[i],
                  (long long)in[i], (long long)dense[i]);
    if (i < 4 && ((size_t)r[i] * es) % 16 != 0)
      return fail(KDA_ERR_ARG, "%s_stride %lld must keep token rows 16-byte aligned", names[i],
                  (long long)in[i]);
  }
  out = kda::InStrides{r[0], r[1], r[2], r[3], r[4]};
  return KDA_OK;
}

// Resolves the optional paged-pool slot stride (0 = dense).
kda_status resolve_slot_stride(int64_t s, int hv, int64_t& out) {
  const int64_t dense = (int64_t)hv * KDA_HEAD_DIM * KDA_HEAD_DIM;
  out = s ? s : dense;
  if (out < dense || out % 8 != 0)
    return fail(KDA_ERR_SHAPE, "state_slot_stride %lld must be 0, or >= %lld and a multiple of 8",
                (long long)s, (long long)dense);
  return KDA_OK;
}

// Gate parameters: both or neither; dt_bias fp32 or bf16; lower_bound in
// [-5, 0], so the step log-decay lower_bound * sigmoid(..) stays in the
// [-5, 0] range that the chunk kernels' block-referenced exponents are built
// for (beyond it the factor between two 16-token block references can
// underflow fp32 while the true coupling is O(1)).
kda_status check_gate(const float* a_log, const void* dt_bias, int32_t dt_dtype, float lb) {
  if ((a_log == nullptr) != (dt_bias == nullptr))
    return fail(KDA_ERR_SHAPE, "A_log and dt_bias must be provided together");
  if (!a_log) return KDA_OK;
  if (dt_dtype != KDA_F32 && dt_dtype != KDA_BF16)
    return fail(KDA_ERR_DTYPE, "dt_bias must be fp32 or bf16");
  if (!(lb >= -5.0f && lb <= 0.0f))
    return fail(KDA_ERR_UNSUPPORTED, "lower_bound must lie in [-5, 0]");
  return KDA_OK;
}

kda::GateArgs gate_of(const float* a_log, const void* dt_bias, int32_t dt_dtype, float lb) {
  kda::GateArgs g;
  g.a_log = a_log;
  g.bias = dt_bias;
  g.bias_bf16 = dt_dtype == KDA_BF16 ? 1 : 0;
  g.lower_bound = lb;
  return g;
}

// Shape and mode checks of the chunked forward (chunk_kda's checks, in the
// terms of this ABI).  Pointers are checked only where the call will read or
// write through them.
kda_status check_chunk(const kda_chunk_args* a, bool need_ptrs) {
  if (!a) return fail(KDA_ERR_ARG, "args is NULL");
  if (a->struct_size != sizeof(kda_chunk_args))
    return fail(KDA_ERR_ARG, "struct_size %zu != sizeof(kda_chunk_args) %zu",
                a->struct_size, sizeof(kda_chunk_args));
  if (a->dtype != KDA_F32 && a->dtype != KDA_BF16 && a->dtype != KDA_F16)
    return fail(KDA_ERR_DTYPE, "unknown dtype %d", a->dtype);
  if (a->num_seqs < 0) return fail(KDA_ERR_SHAPE, "num_seqs must be >= 0");
  if (a->total_tokens < 0) return fail(KDA_ERR_SHAPE, "total_tokens must be >= 0");
  if (a->total_tokens > (int64_t)INT32_MAX)
    return fail(KDA_ERR_UNSUPPORTED, "total_tokens above 2^31-1");
  if (a->hqk <= 0 || a->hv <= 0) return fail(KDA_ERR_SHAPE, "head counts must be > 0");
  if (a->hv % a->hqk != 0)
    return fail(KDA_ERR_SHAPE, "GVA needs hv (%d) divisible by hqk (%d)", a->hv, a->hqk);
  // work items (chunk, value head) are counted in 32 bits
  if ((a->total_tokens / KDA_CHUNK + a->num_seqs) * (int64_t)a->hv > (int64_t)INT32_MAX)
    return fail(KDA_ERR_UNSUPPORTED, "(chunks + sequences) x hv above 2^31-1");
  if (!isfinite(a->scale)) return fail(KDA_ERR_SHAPE, "scale must be finite");
  if (a->cu_seqlens == nullptr) {
    if (a->num_seqs == 0 && a->total_tokens != 0)
      return fail(KDA_ERR_SHAPE, "dense batch with no sequences but %lld tokens",
                  (long long)a->total_tokens);
    if (a->num_seqs > 0 && a->total_tokens % a->num_seqs != 0)
      return fail(KDA_ERR_SHAPE, "dense batch: total_tokens %% num_seqs != 0");
  }
  if (a->state_dtype != KDA_F32 && a->state_dtype != a->dtype)
    return fail(KDA_ERR_DTYPE, "initial/final state must be fp32 or of the input dtype");
  if (a->state_dtype == KDA_F16)
    return fail(KDA_ERR_UNSUPPORTED, "states are stored in fp32 or bf16, not fp16");
  const bool paged = a->state_cache != nullptr;
  if (paged) {
    if (a->initial_state || a->final_state)
      return fail(KDA_ERR_SHAPE, "state_cache replaces initial_state/final_state");
    if (a->num_seqs > 0 && (!a->state_indices || !a->has_initial_state))
      return fail(KDA_ERR_SHAPE, "state_cache needs state_indices and has_initial_state");
    if (a->num_slots <= 0) return fail(KDA_ERR_SHAPE, "num_slots must be > 0");
  } else if (a->state_indices || a->has_initial_state) {
    return fail(KDA_ERR_SHAPE, "state_indices/has_initial_state need a state_cache");
  }
  if (a->path != KDA_PATH_AUTO && a->path != KDA_PATH_STAGED && a->path != KDA_PATH_FUSED &&
      a->path != KDA_PATH_ONCHIP)
    return fail(KDA_ERR_UNSUPPORTED, "unknown path %d", a->path);
  if (a->path == KDA_PATH_ONCHIP && a->dtype != KDA_BF16)
    return fail(KDA_ERR_UNSUPPORTED, "the on-chip path takes bf16 inputs");
  if (a->groups < 0) return fail(KDA_ERR_SHAPE, "groups must be >= 0");
  if (a->max_seqlen < 0) return fail(KDA_ERR_SHAPE, "max_seqlen must be >= 0");
  if (a->groups > 64) return fail(KDA_ERR_UNSUPPORTED, "groups above 64");
  if (a->walk_waves != 0 && a->walk_waves != 2 && a->walk_waves != 4 && a->walk_waves != 8)
    return fail(KDA_ERR_ARG, "walk_waves must be 0, 2, 4 or 8");
  {
    const kda_status gs = check_gate(a->A_log, a->dt_bias, a->dt_bias_dtype, a->lower_bound);
    if (gs != KDA_OK) return gs;
  }
  if ((a->checkpoint_state == nullptr) != (a->checkpoint_offsets == nullptr))
    return fail(KDA_ERR_SHAPE, "checkpoint_state and checkpoint_offsets go together");
  if (a->checkpoint_state) {
    if (a->checkpoint_rows <= 0) return fail(KDA_ERR_SHAPE, "checkpoint_rows must be > 0");
    if (!a->checkpoint_state_indices && a->checkpoint_rows < a->num_seqs)
      return fail(KDA_ERR_SHAPE, "checkpoint_state needs a row per sequence (%d), got %d",
                  a->num_seqs, a->checkpoint_rows);
  }
  if (a->stage_events && (a->num_stage_events < 0 || a->num_stage_events > KDA_NUM_EVENTS))
    return fail(KDA_ERR_ARG, "num_stage_events must be in [0, %d]", KDA_NUM_EVENTS);
  if (need_ptrs && a->total_tokens > 0) {
    if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->out)
      return fail(KDA_ERR_ARG, "q, k, v, g, beta and out must be non-NULL");
  }
  if (misaligned16({a->q, a->k, a->v, a->g, a->out, a->initial_state, a->final_state,
                    a->state_cache, a->checkpoint_state, a->dt_bias}))
    return fail(KDA_ERR_ARG, "tensor base pointers must be 16-byte aligned");
  {
    kda::InStrides st;
    const kda_status ss = resolve_strides(a->q_stride, a->k_stride, a->v_stride, a->g_stride,
                                          a->beta_stride, a->hqk, a->hv, elem_size(a->dtype), st);
    if (ss != KDA_OK) return ss;
    int64_t slot;
    if (paged && resolve_slot_stride(a->state_slot_stride, a->hv, slot) != KDA_OK)
      return KDA_ERR_SHAPE;
    if (!paged && a->state_slot_stride != 0)
      return fail(KDA_ERR_SHAPE, "state_slot_stride needs a state_cache");
  }
  return KDA_OK;
}

int64_t max_chunks_of(const kda_chunk_args* a) {
  return a->total_tokens / KDA_CHUNK + a->num_seqs;
}

// Launch plan of the walk: chunk groups G and waves per walk workgroup (each
// wave owns 16 state columns, so a (sequence, head) spreads over 8 / waves
// workgroups).  The walk is a chain over a sequence's chunks whose length sets
// its time; one walk workgroup is resident per CU (its LDS ring fills most of
// the CU).  Cost in chunk-steps: waves of resident workgroups times chain
// length, with the group scan paying pass one (2x the columns, no outputs),
// G compose steps and pass two over chains G times shorter.  The longest
// sequence's chain is a floor as well: exact for a dense batch, from the
// max_seqlen hint for varlen, else taken as the mean.
struct WalkPlan {
  int groups, waves;
};

WalkPlan plan_walk(const kda_chunk_args* a) {
  const int cap = kda::cu_count_host();  // resident walk workgroups
  const int N = a->num_seqs > 0 ? a->num_seqs : 1;
  const int64_t units = (int64_t)N * a->hv;
  const double nc = (double)max_chunks_of(a) / N;  // chunks per sequence (mean bound)
  const double chain =  // chunks of the longest sequence
      (a->cu_seqlens && a->max_seqlen > 0)
          ? std::min((double)max_chunks_of(a), std::ceil((double)a->max_seqlen / KDA_CHUNK))
          : nc;
  const int waves_opts[3] = {2, 4, 8};
  // time of one chunk step of a workgroup, by waves (measured on MI355X on
  // the dense 4 x 4096 x 16-head prefill: wider workgroups take longer per
  // step; the two-wave bf16 walk has loader waves and warms L2)
  const double cost_bf16[3] = {1.0, 1.45, 2.0}, cost_f32[3] = {1.0, 1.12, 1.55};
  const double* step_cost = a->dtype == KDA_BF16 ? cost_bf16 : cost_f32;
  WalkPlan best = {1, 2};
  double best_cost = 1e300;
  for (int wi = 0; wi < 3; ++wi) {
    const int nw = waves_opts[wi], nvb = 8 / nw;
    if (a->walk_waves > 0 && nw != a->walk_waves) continue;
    for (int G = 1; G <= 64; G *= 2) {
      if (a->groups > 0 && G != a->groups) continue;
      // The group scan fills CUs that the (sequence, head) chains leave
      // idle; with a chain per CU or more it only adds pass one and the
      // compose (measured on the varlen GVA batch, 768 chains: G = 2 took
      // 1.03 ms against 0.89 for the plain walk).
      if (G > 1 && a->groups <= 0 && units >= cap) continue;
      double cost;
      if (G == 1) {
        // With more workgroups than fit at once every CU is busy, and a
        // four-wave bf16 step then costs about as much as an eight-wave one
        // (measured on the varlen GVA batch: 2.0, against 1.45 on the dense
        // prefill, whose four-wave walk leaves half the CUs idle).
        const double rounds = std::ceil((double)(units * nvb) / cap);
        const double c = (a->dtype == KDA_BF16 && nw == 4 && rounds > 1) ? 2.0 : step_cost[wi];
        cost = std::max(rounds * nc, chain) * c;
      } else {
        const double cpg = std::ceil(nc / G);
        const double r2 = std::ceil((double)(units * G * nvb) / cap);
        // pass one walks every group but the last.  bf16: one eight-wave
        // workgroup per group (both column sets, 32 columns a wave; its step
        // measured at 0.5 - 0.8 of an eight-wave pass-two step); fp32: value
        // and transfer workgroups of the pass-two width.
        // Compose takes about four eight-wave steps per group with bf16.
        double p1, comp;
        if (a->dtype == KDA_BF16) {
          p1 = 0.8 * std::ceil((double)(units * (G - 1)) / cap) * step_cost[2] / step_cost[wi];
          comp = 4.0 * G;
        } else {
          p1 = 0.8 * std::ceil((double)(units * (G - 1) * 2 * nvb) / cap);
          comp = G;
        }
        // the group chains (pass one and pass two) have a floor as well
        cost = std::max((p1 + r2) * cpg, 1.8 * std::ceil(chain / G)) * step_cost[wi] + comp;
      }
      if (cost < best_cost * 0.999) {
        best_cost = cost;
        best = {G, nw};
      }
    }
  }
  if (a->groups > 0 && best.groups != a->groups)  // G not a power of 2
    best = {a->groups, a->walk_waves > 0 ? a->walk_waves : 2};
  return best;
}

// The path a call takes: AUTO is the prep-folded staged path, the faster
// of the paths on every workload measured so far (the on-chip path trades
// the intermediates' HBM traffic for a longer serial step per chunk).
int32_t path_of(const kda_chunk_args* a) {
  if (a->path != KDA_PATH_AUTO) return a->path;
  return KDA_PATH_FUSED;
}

// Launch plan of the on-chip path: the chunk groups G.  One chain (a
// (sequence, head) pair, or one group of it) is one 4-wave workgroup.  Two
// walk / pass-two workgroups share a CU (a step of each then costs ~1.3 of a
// lone one's); a pass-one workgroup (twice the state columns) fills a CU and
// its step costs ~1.1.  Cost in chunk steps: waves of resident chains times
// chunks per chain, plus a compose per group; the longest sequence's chain is
// a floor (exact for a dense batch, from the max_seqlen hint for varlen,
// else the mean).
WalkPlan plan_onchip(const kda_chunk_args* a) {
  const int cus = kda::cu_count_host();
  const int N = a->num_seqs > 0 ? a->num_seqs : 1;
  const int64_t units = (int64_t)N * a->hv;
  const double nc = (double)max_chunks_of(a) / N;
  const double chain =
      (a->cu_seqlens && a->max_seqlen > 0)
          ? std::min((double)max_chunks_of(a), std::ceil((double)a->max_seqlen / KDA_CHUNK))
          : nc;
  // time of `chains` chains of `steps` chunk steps on resident workgroups
  auto walk = [&](double chains, double steps, int per_cu, double shared) {
    const double waves = std::ceil(chains / (per_cu * (double)cus));
    const double share = (per_cu > 1 && chains > cus) ? shared : 1.0;
    return waves * steps * share;
  };
  WalkPlan best = {1, 4};
  double best_cost = 1e300;
  for (int G = 1; G <= 64; G *= 2) {
    if (a->groups > 0 && G != a->groups) continue;
    double cost;
    if (G == 1) {
      cost = std::max(walk((double)units, nc, 2, 1.3), chain);
    } else {
      const double cpg = std::ceil(nc / G);
      cost = walk((double)units * (G - 1), cpg, 1, 1.0) * 1.1 +
             walk((double)units * G, cpg, 2, 1.3) + 0.25 * G;
      cost = std::max(cost, 2.1 * std::ceil(chain / G));
    }
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = {G, 4};
    }
  }
  if (a->groups > 0 && best.groups != a->groups) best = {a->groups, 4};  // G not a power of 2
  return best;
}

// Element size of the staged intermediates: bf16 for bf16 inputs, fp32 for
// fp32 and fp16 inputs (fp16 runs on the fp32 kernels).
size_t inter_size(int dtype) { return dtype == KDA_BF16 ? 2 : 4; }

kda_status layout_of(const kda_chunk_args* a, kda_ws_layout* L) {
  memset(L, 0, sizeof(*L));
  const size_t es = inter_size(a->dtype);
  const size_t T = (size_t)a->total_tokens, H = (size_t)a->hv;
  const int64_t mc = max_chunks_of(a);
  const bool onchip = path_of(a) == KDA_PATH_ONCHIP;
  const WalkPlan plan = onchip ? plan_onchip(a) : plan_walk(a);
  const int groups = plan.groups;
  size_t off = 0;
  L->max_chunks = mc;
  L->groups = plan.groups;
  L->walk_waves = plan.waves;
  L->chunk_offsets = off;
  off = align_up(off + sizeof(int32_t) * (2 * (size_t)a->num_seqs + 1), 256);  // + the order
  L->zero = off;
  off = align_up(off + 1024 + 256, 256);  // zero page, WY work counter, longest chunk count
  L->table = off;
  off = align_up(off + 16 * (size_t)mc, 256);
  if (onchip) {
    // no intermediates: the stage regions are empty
    L->qg = L->kg_t = L->decay = L->w = L->u = L->aqk = off;
    L->scan = off;
    if (groups > 1) {
      const size_t planes = (size_t)groups * (size_t)a->num_seqs * H;
      off = align_up(off + planes * 3 * KDA_HEAD_DIM * KDA_HEAD_DIM * sizeof(float), 256);
    }
    L->total = off;
    return KDA_OK;
  }
  L->qg = off;
  off = align_up(off + T * H * KDA_HEAD_DIM * es, 256);
  L->kg_t = off;
  off = align_up(off + (size_t)mc * H * KDA_HEAD_DIM * KDA_CHUNK * es, 256);
  L->decay = off;
  off = align_up(off + (size_t)mc * H * KDA_HEAD_DIM * sizeof(float), 256);
  L->w = off;
  off = align_up(off + T * H * KDA_HEAD_DIM * es, 256);
  L->u = off;
  off = align_up(off + (size_t)mc * H * KDA_HEAD_DIM * KDA_CHUNK * es, 256);
  L->aqk = off;
  off = align_up(off + T * H * KDA_CHUNK * es, 256);
  L->scan = off;
  if (groups > 1) {
    // per (group, sequence, head): transfer P, partial state B, start state
    const size_t planes = (size_t)groups * (size_t)a->num_seqs * H;
    off = align_up(off + planes * 3 * KDA_HEAD_DIM * KDA_HEAD_DIM * sizeof(float), 256);
  }
  L->total = off;
  return KDA_OK;
}

}  // namespace

KDA_API const char* kda_status_str(int32_t s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_SHAPE: return "inconsistent shapes or modes";
    case KDA_ERR_DTYPE: return "unsupported dtype";
    case KDA_ERR_UNSUPPORTED: return "unsupported request";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_HIP: return "HIP launch failure";
    case KDA_ERR_ARG: return "bad argument";
    default: return "unknown status";
  }
}

KDA_API const char* kda_last_error(void) { return g_err; }

KDA_API const char* kda_version(void) { return "kda-mi355x 0.1 (gfx950)"; }

KDA_API kda_status kda_chunk_fwd_workspace_size(const kda_chunk_args* a, size_t* bytes) {
  if (!bytes) return fail(KDA_ERR_ARG, "bytes is NULL");
  kda_status s = check_chunk(a, false);
  if (s != KDA_OK) return s;
  kda_ws_layout L;
  layout_of(a, &L);
  *bytes = L.total;
  return ok();
}

KDA_API kda_status kda_chunk_ws_layout(const kda_chunk_args* a, kda_ws_layout* layout) {
  if (!layout) return fail(KDA_ERR_ARG, "layout is NULL");
  kda_status s = check_chunk(a, false);
  if (s != KDA_OK) return s;
  layout_of(a, layout);
  return ok();
}

namespace {

// KDA_LOG=1 in the environment: one line per chunked-forward call on stderr
// with the launch plan (path, chunk groups, walk width and grids, workspace).
bool log_enabled() {
  static const bool on = [] {
    const char* e = getenv("KDA_LOG");
    return e && e[0] && strcmp(e, "0") != 0;
  }();
  return on;
}

void log_plan(const char* entry, const kda_chunk_args* a, const kda_ws_layout& W) {
  if (!log_enabled()) return;
  static const char* const names[4] = {"auto", "staged", "fused", "onchip"};
  const int32_t p = path_of(a);
  const long long units = (long long)a->num_seqs * a->hv;
  const int G = W.groups, nw = W.walk_waves;
  if (p == KDA_PATH_ONCHIP) {
    fprintf(stderr,
            "kda: %s path=onchip seqs=%d hv=%d tokens=%lld chunks=%lld groups=%d "
            "chains=%lld (4-wave workgroups) workspace=%zu B\n",
            entry, a->num_seqs, a->hv, (long long)a->total_tokens, (long long)W.max_chunks, G,
            units * G, W.total);
    return;
  }
  // Column blocks per (sequence, head) and walk workgroups per pass: 16
  // state columns per compute wave; bf16 pass one walks both column sets in
  // one eight-wave workgroup per group.  Other grids round the (sequence,
  // head[, group]) count up to a multiple of 8.
  auto r8 = [](long long x) { return (x + 7) / 8 * 8; };
  const int bv = 16 * nw, blocks = KDA_HEAD_DIM / bv;
  const long long walk_wgs = r8(units * G) * blocks;
  char scan[160] = "";
  if (G > 1) {
    const bool bf = a->dtype == KDA_BF16;
    const long long p1 = bf ? units * (G - 1) : r8(units * (G - 1)) * 2 * blocks;
    snprintf(scan, sizeof scan, " pass_one_wgs=%lld (%d waves) compose_wgs=%lld", p1,
             bf ? 8 : nw, r8(units) * 8);
  }
  fprintf(stderr,
          "kda: %s path=%s seqs=%d hv=%d tokens=%lld chunks=%lld groups=%d walk_waves=%d "
          "BV=%d walk_wgs=%lld%s wy_wgs=2/CU (persistent) workspace=%zu B\n",
          entry, names[p], a->num_seqs, a->hv, (long long)a->total_tokens,
          (long long)W.max_chunks, G, nw, bv, walk_wgs, scan, W.total);
}

// The chunked forward over an already checked argument set and a workspace
// of at least W.total bytes.
kda_status run_chunk(const kda_chunk_args* a, const kda_ws_layout& W, char* ws) {
  if (a->num_seqs == 0) return ok();
  kda::ChunkLaunch L;
  memset(&L, 0, sizeof(L));
  L.q = a->q; L.k = a->k; L.v = a->v; L.g = a->g; L.beta = a->beta;
  L.cu = a->cu_seqlens;
  L.dtype = a->dtype; L.num_seqs = a->num_seqs; L.hqk = a->hqk; L.hv = a->hv;
  L.use_l2 = a->use_qk_l2norm ? 1 : 0;
  L.total_tokens = a->total_tokens; L.max_chunks = W.max_chunks;
  L.scale = a->scale;
  L.init = a->initial_state; L.fin = a->final_state;
  L.state_bf16 = a->state_dtype == KDA_BF16 ? 1 : 0;
  L.cache = a->state_cache; L.slots = a->state_indices; L.has_init = a->has_initial_state;
  L.num_slots = a->num_slots;
  L.out = a->out;
  L.chunk_offsets = (int32_t*)(ws + W.chunk_offsets);
  L.zero = ws + W.zero;
  L.table = ws + W.table;
  L.qg = ws + W.qg; L.kg_t = ws + W.kg_t; L.decay = (float*)(ws + W.decay);
  L.w = ws + W.w; L.u = ws + W.u; L.aqk = ws + W.aqk;
  L.events = a->stage_events;
  L.num_events = a->stage_events ? a->num_stage_events : 0;
  L.fuse_prep = path_of(a) == KDA_PATH_STAGED ? 0 : 1;
  L.gate = gate_of(a->A_log, a->dt_bias, a->dt_bias_dtype, a->lower_bound);
  L.ckpt = a->checkpoint_state;
  L.ckpt_off = a->checkpoint_offsets;
  L.ckpt_idx = a->checkpoint_state_indices;
  L.ckpt_rows = a->checkpoint_rows;
  resolve_strides(a->q_stride, a->k_stride, a->v_stride, a->g_stride, a->beta_stride, a->hqk,
                  a->hv, elem_size(a->dtype), L.strides);  // checked above
  resolve_slot_stride(a->state_slot_stride, a->hv, L.slot_stride);
  L.groups = W.groups;
  L.walk_waves = W.walk_waves;
  L.scan = L.groups > 1 ? (float*)(ws + W.scan) : nullptr;
  L.stream = a->stream;
  hipError_t e = path_of(a) == KDA_PATH_ONCHIP ? kda::launch_chunk_onchip(L)
                                               : kda::launch_chunk_staged(L);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

// Static scratch of the no-allocation entry point: one copy per device,
// allocated when the code object loads on that device and held until the
// process ends.  Host code never passes `scratch` itself to a kernel (its
// host-side name is not a device address): it resolves the device address
// once per device with hipGetSymbolAddress and uses that.
namespace kda_noalloc {
constexpr size_t SCRATCH_BYTES = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];
}  // namespace kda_noalloc

namespace {
using kda_noalloc::SCRATCH_BYTES;
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];

// The current device's scratch address, resolved on the first call per
// device (with that device current).
kda_status scratch_of_current_device(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES)
    return fail(KDA_ERR_UNSUPPORTED, "device %d beyond the %d devices served", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(kda_noalloc::scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(KDA_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = (char*)g_scratch_ptr[dev];
  return KDA_OK;
}

}  // namespace

KDA_API kda_status kda_chunk_fwd(const kda_chunk_args* a) {
  kda_status s = check_chunk(a, true);
  if (s != KDA_OK) return s;
  kda_ws_layout W;
  layout_of(a, &W);
  if (a->workspace_bytes < W.total || (W.total > 0 && a->workspace == nullptr))
    return fail(KDA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", W.total,
                a->workspace_bytes);
  log_plan("chunk_fwd", a, W);
  return run_chunk(a, W, (char*)a->workspace);
}

KDA_API kda_status kda_chunk_fwd_noalloc(const kda_chunk_args* a) {
  kda_status s = check_chunk(a, true);
  if (s != KDA_OK) return s;
  kda_ws_layout W;
  layout_of(a, &W);
  if (W.total > SCRATCH_BYTES)
    return fail(KDA_ERR_WORKSPACE,
                "this call needs %zu bytes of workspace, beyond the %zu-byte static scratch",
                W.total, SCRATCH_BYTES);
  if (a->num_seqs == 0) return ok();
  log_plan("chunk_fwd_noalloc", a, W);
  char* ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != KDA_OK) return s;
  return run_chunk(a, W, ws);
}


KDA_API kda_status kda_decode(const kda_decode_args* a) {
  if (!a) return fail(KDA_ERR_ARG, "args is NULL");
  if (a->struct_size != sizeof(kda_decode_args))
    return fail(KDA_ERR_ARG, "struct_size %zu != sizeof(kda_decode_args) %zu",
                a->struct_size, sizeof(kda_decode_args));
  if (a->dtype != KDA_F32 && a->dtype != KDA_BF16 && a->dtype != KDA_F16)
    return fail(KDA_ERR_DTYPE, "unknown dtype %d", a->dtype);
  if (a->n < 0) return fail(KDA_ERR_SHAPE, "n must be >= 0");
  if (a->hqk <= 0 || a->hv <= 0) return fail(KDA_ERR_SHAPE, "head counts must be > 0");
  if (a->hv % a->hqk != 0)
    return fail(KDA_ERR_SHAPE, "GVA needs hv (%d) divisible by hqk (%d)", a->hv, a->hqk);
  if (!isfinite(a->scale)) return fail(KDA_ERR_SHAPE, "scale must be finite");
  if (a->num_slots <= 0) return fail(KDA_ERR_SHAPE, "state pool must have at least one slot");
  if (!a->state_indices && a->num_slots < a->n)
    return fail(KDA_ERR_SHAPE, "state pool must contain at least %d slots, got %d", a->n,
                a->num_slots);
  if ((size_t)a->n * (size_t)a->hv > 0x7fffffffu)
    return fail(KDA_ERR_UNSUPPORTED, "n * hv above 2^31-1");
  {
    const kda_status gs = check_gate(a->A_log, a->dt_bias, a->dt_bias_dtype, a->lower_bound);
    if (gs != KDA_OK) return gs;
  }
  if (a->state_dtype != KDA_F32 && a->state_dtype != KDA_BF16)
    return fail(KDA_ERR_DTYPE, "state_cache must be fp32 or bf16");
  if (misaligned16({a->q, a->k, a->v, a->g, a->out, a->state_cache, a->dt_bias}))
    return fail(KDA_ERR_ARG, "tensor base pointers must be 16-byte aligned");
  kda::InStrides strides;
  {
    const kda_status ss = resolve_strides(a->q_stride, a->k_stride, a->v_stride, a->g_stride,
                                          a->beta_stride, a->hqk, a->hv, elem_size(a->dtype),
                                          strides);
    if (ss != KDA_OK) return ss;
  }
  int64_t slot_stride;
  if (resolve_slot_stride(a->state_slot_stride, a->hv, slot_stride) != KDA_OK)
    return KDA_ERR_SHAPE;
  if (a->tokens < 0 || a->tokens > 8)
    return fail(KDA_ERR_UNSUPPORTED, "tokens per request must lie in [0, 8], got %d", a->tokens);
  const int T = a->tokens > 1 ? a->tokens : 1;
  if (a->state_index_cols < 0) return fail(KDA_ERR_SHAPE, "state_index_cols must be >= 0");
  if (a->state_index_cols > 0 && !a->state_indices)
    return fail(KDA_ERR_SHAPE, "state_index_cols needs state_indices");
  if (a->state_index_cols > 0 && a->state_index_cols < T)
    return fail(KDA_ERR_SHAPE, "state_indices needs at least %d columns, got %d", T,
                a->state_index_cols);
  if ((T > 1 || a->num_accepted_tokens) && a->state_index_cols == 0)
    return fail(KDA_ERR_SHAPE,
                "multi-token or speculative decode needs [n, T] state_indices");
  if ((size_t)a->n * (size_t)T * (size_t)a->hv > 0x7fffffffu)
    return fail(KDA_ERR_UNSUPPORTED, "n * tokens * hv above 2^31-1");
  if (a->n == 0) return ok();
  if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->out || !a->state_cache)
    return fail(KDA_ERR_ARG, "q, k, v, g, beta, out and state_cache must be non-NULL");
  kda::DecodeLaunch L;
  L.q = a->q; L.k = a->k; L.v = a->v; L.g = a->g; L.beta = a->beta;
  L.cache = a->state_cache; L.idx = a->state_indices; L.out = a->out;
  L.state_bf16 = a->state_dtype == KDA_BF16 ? 1 : 0;
  L.dtype = a->dtype; L.n = a->n; L.hqk = a->hqk; L.hv = a->hv;
  L.use_l2 = a->use_qk_l2norm ? 1 : 0; L.num_slots = a->num_slots; L.scale = a->scale;
  L.stream = a->stream;
  L.gate = gate_of(a->A_log, a->dt_bias, a->dt_bias_dtype, a->lower_bound);
  L.tokens = T;
  L.cols = a->state_index_cols;
  L.accepted = a->num_accepted_tokens;
  L.strides = strides;
  L.slot_stride = slot_stride;
  hipError_t e = kda::launch_decode(L);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

KDA_API kda_status kda_verify(const kda_verify_args* a) {
  if (!a) return fail(KDA_ERR_ARG, "args is NULL");
  if (a->struct_size != sizeof(kda_verify_args))
    return fail(KDA_ERR_ARG, "struct_size %zu != sizeof(kda_verify_args) %zu", a->struct_size,
                sizeof(kda_verify_args));
  if (a->dtype != KDA_F32 && a->dtype != KDA_BF16 && a->dtype != KDA_F16)
    return fail(KDA_ERR_DTYPE, "unknown dtype %d", a->dtype);
  if (a->n < 0) return fail(KDA_ERR_SHAPE, "n must be >= 0");
  if (a->hqk <= 0 || a->hv <= 0) return fail(KDA_ERR_SHAPE, "head counts must be > 0");
  if (a->hv % a->hqk != 0)
    return fail(KDA_ERR_SHAPE, "GVA needs hv (%d) divisible by hqk (%d)", a->hv, a->hqk);
  if (a->window < 1 || a->window > 8)
    return fail(KDA_ERR_SHAPE, "window must lie in [1, 8], got %d", a->window);
  if (!isfinite(a->scale)) return fail(KDA_ERR_SHAPE, "scale must be finite");
  if (a->num_slots <= 0) return fail(KDA_ERR_SHAPE, "state pool must have at least one slot");
  if (a->state_dtype != KDA_F32 && a->state_dtype != KDA_BF16)
    return fail(KDA_ERR_DTYPE, "state_cache must be fp32 or bf16");
  {
    const kda_status gs = check_gate(a->A_log, a->dt_bias, a->dt_bias_dtype, a->lower_bound);
    if (gs != KDA_OK) return gs;
  }
  if ((size_t)a->n * (size_t)a->hv > 0x7fffffffu)
    return fail(KDA_ERR_UNSUPPORTED, "n * hv above 2^31-1");
  if (misaligned16({a->q, a->k, a->v, a->g, a->out, a->state_cache, a->kg, a->corr, a->dt_bias}))
    return fail(KDA_ERR_ARG, "tensor base pointers must be 16-byte aligned");
  kda::InStrides strides;
  {
    const kda_status ss = resolve_strides(a->q_stride, a->k_stride, a->v_stride, a->g_stride,
                                          a->beta_stride, a->hqk, a->hv, elem_size(a->dtype),
                                          strides);
    if (ss != KDA_OK) return ss;
  }
  int64_t slot_stride;
  if (resolve_slot_stride(a->state_slot_stride, a->hv, slot_stride) != KDA_OK)
    return KDA_ERR_SHAPE;
  if (a->n == 0) return ok();
  if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->query_start || !a->state_cache ||
      !a->state_indices || !a->corr || !a->kg || !a->out)
    return fail(KDA_ERR_ARG,
                "q, k, v, g, beta, query_start, state_cache, state_indices, corr, kg and out "
                "must be non-NULL");
  kda::VerifyLaunch L;
  L.q = a->q; L.k = a->k; L.v = a->v; L.g = a->g; L.beta = a->beta;
  L.query_start = a->query_start;
  L.cache = a->state_cache; L.state_bf16 = a->state_dtype == KDA_BF16 ? 1 : 0;
  L.idx = a->state_indices; L.corr = a->corr; L.kg = a->kg; L.out = a->out;
  L.dtype = a->dtype; L.n = a->n; L.hqk = a->hqk; L.hv = a->hv; L.window = a->window;
  L.use_l2 = a->use_qk_l2norm ? 1 : 0; L.num_slots = a->num_slots; L.scale = a->scale;
  L.gate = gate_of(a->A_log, a->dt_bias, a->dt_bias_dtype, a->lower_bound);
  L.strides = strides; L.slot_stride = slot_stride; L.stream = a->stream;
  hipError_t e = kda::launch_verify(L);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

KDA_API kda_status kda_commit(const kda_commit_args* a) {
  if (!a) return fail(KDA_ERR_ARG, "args is NULL");
  if (a->struct_size != sizeof(kda_commit_args))
    return fail(KDA_ERR_ARG, "struct_size %zu != sizeof(kda_commit_args) %zu", a->struct_size,
                sizeof(kda_commit_args));
  if (a->dtype != KDA_F32 && a->dtype != KDA_BF16 && a->dtype != KDA_F16)
    return fail(KDA_ERR_DTYPE, "unknown dtype %d", a->dtype);
  if (a->n < 0) return fail(KDA_ERR_SHAPE, "n must be >= 0");
  if (a->hv <= 0) return fail(KDA_ERR_SHAPE, "head count must be > 0");
  if (a->window < 1 || a->window > 8)
    return fail(KDA_ERR_SHAPE, "window must lie in [1, 8], got %d", a->window);
  if (a->num_slots <= 0) return fail(KDA_ERR_SHAPE, "state pool must have at least one slot");
  if (a->state_dtype != KDA_F32 && a->state_dtype != KDA_BF16)
    return fail(KDA_ERR_DTYPE, "state_cache must be fp32 or bf16");
  {
    const kda_status gs = check_gate(a->A_log, a->dt_bias, a->dt_bias_dtype, a->lower_bound);
    if (gs != KDA_OK) return gs;
  }
  if ((size_t)a->n * (size_t)a->hv > 0x7fffffffu)
    return fail(KDA_ERR_UNSUPPORTED, "n * hv above 2^31-1");
  if (misaligned16({a->state_cache, a->kg, a->corr, a->dt_bias}))
    return fail(KDA_ERR_ARG, "tensor base pointers must be 16-byte aligned");
  int64_t slot_stride;
  if (resolve_slot_stride(a->state_slot_stride, a->hv, slot_stride) != KDA_OK)
    return KDA_ERR_SHAPE;
  if (a->n == 0) return ok();
  if (!a->state_cache || !a->state_indices || !a->num_accepted_tokens || !a->corr || !a->kg)
    return fail(KDA_ERR_ARG,
                "state_cache, state_indices, num_accepted_tokens, corr and kg must be non-NULL");
  kda::CommitLaunch L;
  L.cache = a->state_cache; L.state_bf16 = a->state_dtype == KDA_BF16 ? 1 : 0;
  L.idx = a->state_indices; L.accepted = a->num_accepted_tokens;
  L.corr = a->corr; L.kg = a->kg;
  L.dtype = a->dtype; L.n = a->n; L.hv = a->hv; L.window = a->window;
  L.use_l2 = a->use_qk_l2norm ? 1 : 0; L.num_slots = a->num_slots;
  L.gate = gate_of(a->A_log, a->dt_bias, a->dt_bias_dtype, a->lower_bound);
  L.slot_stride = slot_stride; L.stream = a->stream;
  hipError_t e = kda::launch_commit(L);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}
