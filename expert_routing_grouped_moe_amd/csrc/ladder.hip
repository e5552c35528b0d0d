// Graph ladder: one captured HIP graph of the whole layer per batch-size bucket, so that a decode
// loop whose batch width changes from step to step replays a graph instead of launching kernels
// (zonos2.cpp INTERNALS, "Performance": the decode graph is captured once and replayed). Host code
// only; every graph is a capture of moe_layer_forward itself. A bucket larger than the step's T
// also routes the padding rows, so when the caller wants expert counts they are recounted from the
// first T rows' ids after the replay.
#include <hip/hip_runtime.h>

#include <cstring>
#include <new>

#include "kernels.hpp"
#include "moe.h"

struct moe_graph_ladder {
  int n;
  int32_t bucket[MOE_LADDER_MAX_BUCKETS];
  hipGraphExec_t exec[MOE_LADDER_MAX_BUCKETS];
  const int32_t* ids[MOE_LADDER_MAX_BUCKETS];  // where bucket i's graph leaves the expert ids
  int32_t* counts;                             // the caller's expert_counts, or NULL
  int k, E;
};

namespace {

void release(moe_graph_ladder* l) {
  for (int i = 0; i < l->n; ++i)
    if (l->exec[i]) (void)hipGraphExecDestroy(l->exec[i]);
  delete l;
}

}  // namespace

extern "C" {

int moe_ladder_create(const moe_layer_args* a, const int32_t* buckets, int n_buckets, void* ws,
                      size_t ws_bytes, void* stream, moe_graph_ladder** out) {
  if (!a || !buckets || !out) return MOE_ERR_NULL;
  *out = nullptr;
  if (a->struct_size < MOE_LAYER_ARGS_V1_SIZE || a->struct_size > sizeof(moe_layer_args))
    return MOE_ERR_UNSUPPORTED;
  if (n_buckets < 1 || n_buckets > MOE_LADDER_MAX_BUCKETS) return MOE_ERR_SHAPE;
  for (int i = 0; i < n_buckets; ++i) {
    if (buckets[i] < 1 || buckets[i] > a->T) return MOE_ERR_SHAPE;
    if (i > 0 && buckets[i] <= buckets[i - 1]) return MOE_ERR_SHAPE;
  }
  // capture needs a stream of its own, not one already being captured
  if (!stream) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) return MOE_ERR_HIP;
  if (cs != hipStreamCaptureStatusNone) return MOE_ERR_UNSUPPORTED;

  moe_graph_ladder* l = new (std::nothrow) moe_graph_ladder;
  if (!l) return MOE_ERR_HIP;
  l->n = 0;
  l->counts = a->expert_counts;
  l->k = a->k;
  l->E = a->E;
  moe_layer_args ab;
  std::memset(&ab, 0, sizeof(ab));
  std::memcpy(&ab, a, a->struct_size);
  ab.prof_events = nullptr;  // graphs replay kernels only
  for (int i = 0; i < n_buckets; ++i) {
    ab.T = buckets[i];
    if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess) {
      release(l);
      return MOE_ERR_HIP;
    }
    const int st = moe_layer_forward(&ab, ws, ws_bytes, stream);
    hipGraph_t g = nullptr;
    const hipError_t ec = hipStreamEndCapture(s, &g);
    if (st != MOE_OK || ec != hipSuccess || !g) {
      if (g) (void)hipGraphDestroy(g);
      release(l);
      return st != MOE_OK ? st : MOE_ERR_HIP;
    }
    hipGraphExec_t exec = nullptr;
    const hipError_t ei = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (ei != hipSuccess) {
      release(l);
      return MOE_ERR_HIP;
    }
    l->bucket[i] = buckets[i];
    l->exec[i] = exec;
    l->ids[i] = a->topk_ids ? a->topk_ids
                            : reinterpret_cast<const int32_t*>(
                                  static_cast<const char*>(ws) +
                                  moe::layer_ids_offset(buckets[i], a->d, a->E, a->H, a->k,
                                                        a->dtype));
    l->n = i + 1;
  }
  *out = l;
  return MOE_OK;
}

int moe_ladder_run(const moe_graph_ladder* l, int T, void* stream, int32_t* bucket_out) {
  if (!l) return MOE_ERR_NULL;
  if (T < 1 || T > l->bucket[l->n - 1]) return MOE_ERR_SHAPE;
  int i = 0;
  while (l->bucket[i] < T) ++i;
  if (bucket_out) *bucket_out = l->bucket[i];
  (void)hipGetLastError();
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipGraphLaunch(l->exec[i], s) != hipSuccess) return MOE_ERR_HIP;
  // the graph counted the padding rows T..b-1 as well
  if (l->counts && l->bucket[i] > T &&
      moe::launch_counts(l->ids[i], T * l->k, l->E, l->counts, s) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

void moe_ladder_destroy(moe_graph_ladder* l) {
  if (l) release(l);
}

}  // extern "C"
