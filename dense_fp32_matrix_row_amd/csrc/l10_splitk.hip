// l10_splitk.hip -- split K for problems too small in M x N to fill the
// GPU: a matrix-core tile kernel (level 10's 64 x 64 assembly loop, or any
// tile hip_sgemm_tile_split names) with each tile's K range cut into slices
// that run as separate work items, then one reduction kernel.
//
// The technique is the one the pages describe behind the vendor library's
// small-size advantage ([GEMM2], size-sweep section: at 256 the vendor calls
// a tiled GEMM plus a reduce kernel; each block computes part of the K sum
// for its C block, the partial sums need extra storage, a reduce kernel adds
// them).  At 512 x 512 x 8192 the 64 x 64 tile grid has 64 tiles for 256
// CUs; eight slices of K make 512 work items (two per CU).
//
// Determinism: the number of slices depends only on the shape, every slice
// stores its float32 sums into its own plane of the workspace (no atomics),
// and the reduction adds the planes in slice order 0, 1, ..., S-1 before
// the alpha/beta epilogue.  Results are bit-reproducible; they differ from
// the unsplit tile in the last bits (one float32 chain per slice instead of
// one for the whole K), within the same rounding bound.
//
// Workspace: S x M x N floats per call, taken from a stream-ordered memory
// pool that the library creates per device on first use and keeps for the
// life of the process (release threshold: never), allocated and freed on the
// caller's stream around the two kernels.  Concurrent calls on other
// streams therefore never share a workspace.  On a stream being captured
// into a graph the pool is not touched (it can be neither created nor
// configured during a capture): the workspace is then a stream-ordered
// allocation from the device's default pool, which the capture records as
// a graph memory node.
//
// The no-allocation entry point (hip_sgemm_ex_noalloc) takes the workspace
// from `scratch` instead: a fixed array in each device's memory, loaded
// with the library's code object and kept until the process ends.  Host
// code reaches it only through the address hipGetSymbolAddress gives for
// a device while that device is current (looked up once per device); the
// array's name itself is a host-side stand-in, not a device address.
//
// Both workspaces belong to the device the caller's stream runs on, which
// need not be the calling thread's current device.  Every element a call
// reads back from its planes it has written first, so nothing needs
// clearing between calls; calls that overlap on one device share the
// array and race.
#include <mutex>

#include "sgemm.h"
#include "sgemm_internal.h"

namespace sgemm {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_pool_mutex;
hipMemPool_t g_pools[kMaxDevices];

constexpr int64_t kScratchFloats = SGEMM_NOALLOC_WORKSPACE_BYTES / int64_t(sizeof(float));
static __device__ __align__(256) float scratch[kScratchFloats];
std::mutex g_scratch_mutex;
float* g_scratch[kMaxDevices];  // scratch's device address, per device

// The device whose queue a stream feeds (the current device for the null
// stream).
hipError_t stream_device(hipStream_t s, int* dev) {
  if (s == nullptr) return hipGetDevice(dev);
  hipDevice_t d = 0;
  const hipError_t e = hipStreamGetDevice(s, &d);
  if (e == hipSuccess) *dev = d;
  return e;
}

hipError_t scratch_for_device(int dev, float** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    // the symbol's address is the current device's copy: make dev current
    // for the lookup, then give the calling thread its device back
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

hipError_t pool_for_device(int dev, hipMemPool_t* out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  hipError_t e = hipSuccess;
  std::lock_guard<std::mutex> lock(g_pool_mutex);
  if (g_pools[dev] == nullptr) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    e = hipMemPoolCreate(&pool, &props);
    if (e != hipSuccess) return e;
    uint64_t keep = UINT64_MAX;  // keep freed blocks cached for reuse
    e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) {
      (void)hipMemPoolDestroy(pool);
      return e;
    }
    g_pools[dev] = pool;
  }
  *out = g_pools[dev];
  return hipSuccess;
}

// C[i][j] <- alpha * (((W_0 + W_1) + W_2) + ... + W_{S-1})[i][j] + beta * C[i][j],
// four adjacent columns per thread (128-bit accesses where whole).
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ ws,
                                                       int64_t splits, int M, int N,
                                                       float alpha, float beta,
                                                       float* __restrict__ C, int64_t ldc,
                                                       int64_t groups_per_row,
                                                       int64_t ngroups) {
  const int64_t plane = int64_t(M) * N;
  for (int64_t g = int64_t(blockIdx.x) * 256 + threadIdx.x; g < ngroups;
       g += int64_t(gridDim.x) * 256) {
    const int64_t row = g / groups_per_row, col = 4 * (g % groups_per_row);
    const float* w = ws + row * N;
    float4 sum = load4(w, col, N, true);
    for (int64_t s = 1; s < splits; ++s) {
      const float4 v = load4(w + s * plane, col, N, true);
      sum.x += v.x;
      sum.y += v.y;
      sum.z += v.z;
      sum.w += v.w;
    }
    store4(C + row * ldc + col, col, N, sum, alpha, beta);
  }
}

hipError_t launch_reduce(const float* ws, int64_t splits, const Problem& p, hipStream_t s) {
  const int64_t groups_per_row = ceil_div(p.N, 4);
  const int64_t ngroups = int64_t(p.M) * groups_per_row;
  const int64_t want = ceil_div(ngroups, 256);
  const int64_t blocks = want < 8192 ? want : 8192;  // grid-stride beyond
  hipLaunchKernelGGL(k_splitk_reduce, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, ws,
                     splits, p.M, p.N, p.alpha, p.beta, p.C, p.ldc, groups_per_row, ngroups);
  return hipGetLastError();
}

// Workspace, then launch_split(ws) (the split tile kernel), then the
// reduction; the workspace from the source w.
template <class F>
hipError_t splitk_with(F launch_split, int64_t k_split, const Problem& p, hipStream_t s,
                       Workspace w) {
  const int64_t splits = ceil_div(p.K, k_split);
  const size_t bytes = size_t(splits) * size_t(p.M) * size_t(p.N) * sizeof(float);
  if (w == Workspace::kStatic) {
    // the fixed array: no allocation, no release
    if (bytes > size_t(SGEMM_NOALLOC_WORKSPACE_BYTES)) return hipErrorInvalidValue;
    float* ws = nullptr;
    int dev = 0;
    hipError_t e = stream_device(s, &dev);
    if (e == hipSuccess) e = scratch_for_device(dev, &ws);
    if (e != hipSuccess) return e;
    e = launch_split(ws);
    if (e == hipSuccess) e = launch_reduce(ws, splits, p, s);
    return e;
  }
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &capture);
  if (e != hipSuccess) return e;
  void* ws = nullptr;
  if (capture == hipStreamCaptureStatusActive) {
    e = hipMallocAsync(&ws, bytes, s);
  } else {
    hipMemPool_t pool = nullptr;
    int dev = 0;
    e = stream_device(s, &dev);
    if (e == hipSuccess) e = pool_for_device(dev, &pool);
    if (e != hipSuccess) return e;
    e = hipMallocFromPoolAsync(&ws, bytes, pool, s);
  }
  if (e != hipSuccess) return e;
  e = launch_split(static_cast<float*>(ws));
  if (e == hipSuccess) e = launch_reduce(static_cast<const float*>(ws), splits, p, s);
  const hipError_t f = hipFreeAsync(ws, s);
  return e != hipSuccess ? e : f;
}

}  // namespace

int64_t static_workspace_bytes() { return SGEMM_NOALLOC_WORKSPACE_BYTES; }

hipError_t launch_splitk(Shape shape, int64_t k_split, const Problem& p, hipStream_t s,
                         Workspace w) {
  return splitk_with([&](float* ws) { return launch_tiles_split(shape, p, k_split, ws, s); },
                     k_split, p, s, w);
}

hipError_t launch_splitk_fn(SplitLaunchFn fn, int64_t k_split, const Problem& p, hipStream_t s) {
  return splitk_with([&](float* ws) { return fn(p, k_split, ws, s); }, k_split, p, s,
                     Workspace::kPool);
}

}  // namespace sgemm
