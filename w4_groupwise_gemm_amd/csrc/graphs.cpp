// Per-verify-width graph set: the launch-overhead removal of a decode step.
//
// A speculative decode round calls the same projections at a handful of token widths
// (concurrency x (draft + 1)), and at one stream the kernels are short enough that the gaps
// between launches and each kernel's ramp-up and drain are a large share of the step (ninfer-3080
// performance notes, "What is left at C1": the cost is mostly ramp-up and drain at the kernel
// boundaries; Kernarc, "One decode step, top to silicon": one captured graph per verify width).
// Every compute call of this library is capturable (validation is synchronous, nothing is
// allocated, exactly one or two kernels are enqueued), so a caller records the calls of one step
// at one width once and replays the instantiated graph at every later step of that width.
//
// The set maps width -> instantiated graph.  Capture uses the relaxed capture mode: the
// library's own host calls during capture (the device query of its one-time gfx950 check) are
// not stream work and stay allowed.  Buffers named by the captured calls must stay
// allocated, at the same addresses, for as long as the graph is replayed.
#include <hip/hip_runtime.h>

#include <map>
#include <new>
#include <mutex>

#include "../../include/w4gemm.h"

struct w4_graph_set {
  std::mutex mu;
  std::map<int, hipGraphExec_t> exec;  // width -> instantiated graph
  int capturing = -1;                  // width being captured, -1 if none
  hipStream_t capture_stream = nullptr;
};

extern "C" w4_graph_set* w4_graph_set_create(void) { return new (std::nothrow) w4_graph_set(); }

extern "C" int w4_graph_set_begin(w4_graph_set* set, int width, void* stream) {
  if (!set || width < 0 || !stream) return W4_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(set->mu);
  if (set->capturing >= 0) return W4_ERR_INVALID_ARG;  // one capture at a time per set
  if (set->exec.count(width)) return W4_ERR_INVALID_ARG;  // already recorded
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipStreamBeginCapture(st, hipStreamCaptureModeRelaxed) != hipSuccess) return W4_ERR_DEVICE;
  set->capturing = width;
  set->capture_stream = st;
  return W4_OK;
}

extern "C" int w4_graph_set_end(w4_graph_set* set, int width, void* stream) {
  if (!set || !stream) return W4_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(set->mu);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (set->capturing != width || set->capture_stream != st) return W4_ERR_INVALID_ARG;
  set->capturing = -1;
  set->capture_stream = nullptr;
  hipGraph_t g = nullptr;
  if (hipStreamEndCapture(st, &g) != hipSuccess || !g) return W4_ERR_LAUNCH;
  hipGraphExec_t e = nullptr;
  const hipError_t err = hipGraphInstantiate(&e, g, nullptr, nullptr, 0);
  hipGraphDestroy(g);
  if (err != hipSuccess || !e) return W4_ERR_LAUNCH;
  set->exec[width] = e;
  return W4_OK;
}

extern "C" int w4_graph_set_launch(w4_graph_set* set, int width, void* stream) {
  if (!set) return W4_ERR_INVALID_ARG;
  hipGraphExec_t e = nullptr;
  {
    std::lock_guard<std::mutex> lock(set->mu);
    auto it = set->exec.find(width);
    if (it == set->exec.end()) return W4_ERR_DOMAIN;
    e = it->second;
  }
  return hipGraphLaunch(e, static_cast<hipStream_t>(stream)) == hipSuccess ? W4_OK : W4_ERR_LAUNCH;
}

extern "C" int w4_graph_set_has(w4_graph_set* set, int width) {
  if (!set) return 0;
  std::lock_guard<std::mutex> lock(set->mu);
  return set->exec.count(width) ? 1 : 0;
}

extern "C" void w4_graph_set_destroy(w4_graph_set* set) {
  if (!set) return;
  {
    std::lock_guard<std::mutex> lock(set->mu);
    for (auto& kv : set->exec) hipGraphExecDestroy(kv.second);
    set->exec.clear();
  }
  delete set;
}
