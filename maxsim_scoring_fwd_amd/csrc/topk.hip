// libmaxsim top-k entry points (include/maxsim.h): the best k documents of each score row.
#include <hip/hip_runtime.h>

#include <mutex>
#include <unordered_map>

#include "host_common.hpp"
#include "topk_kernel.hpp"

using namespace maxsim;

// Scratch memory of maxsim_topk_no_alloc: the sorted runs (or kept keys) between passes.
// Each GPU the library runs on holds its own copy until the process ends. Host code never
// passes this name to a kernel (on the host it is only a stand-in for the symbol): it uses
// the device address that hipGetSymbolAddress returns for the current device.
constexpr size_t TOPK_SCRATCH_BYTES = size_t(8) << 20;
static __device__ __align__(256) uint64_t scratch[TOPK_SCRATCH_BYTES / sizeof(uint64_t)];

namespace {

// Device address of `scratch` on the current device, looked up once per device.
int scratch_address(void **ptr) {
  static std::mutex mu;
  static std::unordered_map<int, void *> addr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MAXSIM_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return MAXSIM_ERR_DEVICE;
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return MAXSIM_OK;
}

int64_t chunks_of(int64_t count) { return (count + TOPK_CHUNK - 1) / TOPK_CHUNK; }

bool topk_args_ok(int64_t n, int rows, int k) {
  return n >= 1 && n < ((int64_t)1 << 31) && rows >= 1 && rows <= 65535 && k >= 1 &&
         k <= TOPK_MAX_K;
}

// k <= 128: pass 1 leaves one sorted run per 2048 scores; merge passes reduce up to 64 runs
// per workgroup until one run per row remains, whose first k entries are the result.
// ws holds the runs of pass 1 and, when it takes two or more merge passes, of the first
// merge pass; later passes alternate between the two regions.
int topk_runs(const float *scores, int64_t n, int rows, int k, float *out_scores,
              int32_t *out_index, uint64_t *ws, hipStream_t st) {
  const int64_t c1 = (n + RUN_CHUNK - 1) / RUN_CHUNK;
  uint64_t *buf[2] = {ws, ws ? ws + c1 * RUN * rows : nullptr};
  TopkRunArgs a{scores, n, nullptr, 0, c1 > 1 ? buf[0] : nullptr, k, out_scores, out_index};
  hipLaunchKernelGGL(topk_runs_kernel, dim3((unsigned)c1, (unsigned)rows), dim3(RUN_THREADS), 0,
                     st, a);
  if (hipGetLastError() != hipSuccess) return MAXSIM_ERR_LAUNCH;
  int64_t runs = c1;
  for (int pass = 0; runs > 1; pass++) {
    const int64_t groups = (runs + RUN_FANIN - 1) / RUN_FANIN;
    a.in_runs = buf[pass & 1];
    a.n_runs = runs;
    a.out_runs = groups > 1 ? buf[(pass + 1) & 1] : nullptr;
    hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)groups, (unsigned)rows),
                       dim3(RUN_THREADS), 0, st, a);
    if (hipGetLastError() != hipSuccess) return MAXSIM_ERR_LAUNCH;
    runs = groups;
  }
  return MAXSIM_OK;
}

}  // namespace

extern "C" {

size_t maxsim_topk_workspace_size(int64_t n, int rows, int k) {
  if (!topk_args_ok(n, rows, k)) return 0;
  if (k <= RUN_MAX_K) {
    // runs of the first pass, and of the second where more than one merge pass is needed
    const int64_t c1 = (n + RUN_CHUNK - 1) / RUN_CHUNK;
    if (c1 <= 1) return 0;
    const int64_t c2 = (c1 + RUN_FANIN - 1) / RUN_FANIN;
    return (size_t)(c1 + (c2 > 1 ? c2 : 0)) * RUN * (size_t)rows * sizeof(uint64_t);
  }
  const int64_t c1 = chunks_of(n);
  if (c1 <= 1) return 0;
  const int64_t c2 = chunks_of(c1 * k);
  return (size_t)(c1 + (c2 > 1 ? c2 : 0)) * (size_t)k * (size_t)rows * sizeof(uint64_t);
}

int maxsim_topk(const float *scores, int64_t n, int rows, int k, float *out_scores,
                int32_t *out_index, void *workspace, size_t workspace_bytes, void *stream) {
  if (!topk_args_ok(n, rows, k)) return MAXSIM_ERR_SHAPE;
  if (!scores || !out_scores || !out_index) return MAXSIM_ERR_NULL;
  if (!aligned(scores, 4) || !aligned(out_scores, 4) || !aligned(out_index, 4) ||
      (workspace && !aligned(workspace, 8)))
    return MAXSIM_ERR_ALIGN;
  const size_t need = maxsim_topk_workspace_size(n, rows, k);
  if (need > 0 && (!workspace || workspace_bytes < need)) return workspace ? MAXSIM_ERR_SHAPE
                                                                           : MAXSIM_ERR_NULL;
  DeviceInfo di;
  int rc = current_device(di);
  if (rc != MAXSIM_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (k <= RUN_MAX_K) return topk_runs(scores, n, rows, k, out_scores, out_index,
                                       (uint64_t *)workspace, st);
  const int64_t c1 = chunks_of(n);
  uint64_t *buf[2] = {(uint64_t *)workspace, (uint64_t *)workspace + (c1 > 1 ? c1 * k * rows : 0)};
  TopkLevelArgs a{scores, nullptr, n, n, k, nullptr, 0, out_scores, out_index, scores, n};
  for (int level = 0;; level++) {
    const int64_t chunks = chunks_of(a.count);
    if (chunks == 1) {  // the final chunk: sorted top-k out
      a.out_keys = nullptr;
      hipLaunchKernelGGL(topk_level_kernel, dim3(1, (unsigned)rows), dim3(TOPK_THREADS), 0, st, a);
      return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
    }
    a.out_keys = buf[level & 1];
    a.out_stride = chunks * k;
    hipLaunchKernelGGL(topk_level_kernel, dim3((unsigned)chunks, (unsigned)rows),
                       dim3(TOPK_THREADS), 0, st, a);
    if (hipGetLastError() != hipSuccess) return MAXSIM_ERR_LAUNCH;
    a.scores = nullptr;
    a.in_keys = a.out_keys;
    a.count = chunks * k;
    a.in_stride = a.out_stride;
  }
}

int maxsim_topk_no_alloc(const float *scores, int64_t n, int rows, int k, float *out_scores,
                         int32_t *out_index, void *stream) {
  if (!topk_args_ok(n, rows, k)) return MAXSIM_ERR_SHAPE;
  if (maxsim_topk_workspace_size(n, rows, k) > TOPK_SCRATCH_BYTES) return MAXSIM_ERR_SCRATCH;
  if (!scores || !out_scores || !out_index) return MAXSIM_ERR_NULL;
  DeviceInfo di;
  int rc = current_device(di);
  if (rc != MAXSIM_OK) return rc;
  void *ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != MAXSIM_OK) return rc;
  return maxsim_topk(scores, n, rows, k, out_scores, out_index, ws, TOPK_SCRATCH_BYTES, stream);
}

size_t maxsim_topk_scratch_bytes(void) { return TOPK_SCRATCH_BYTES; }

}  // extern "C"
