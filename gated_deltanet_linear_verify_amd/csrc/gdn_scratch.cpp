// gdn_scratch.cpp - the readout scratch of the row-split verify: one device buffer per (device,
// stream), so that calls on different streams never share one.  A buffer is allocated on the first
// split launch on its stream, outside stream capture; under capture only a buffer reserved before
// the capture began is used (gdn_graph reserves one for its capture stream and keeps it for the
// graph's lifetime), and without one the launcher takes the unsplit path.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <utility>

#include "gdn_internal.h"

namespace gdn {
namespace {

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, void *> g_bufs;

bool capturing(hipStream_t st)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) return true;  // unknown: do not allocate
    return cs != hipStreamCaptureStatusNone;
}

}  // namespace

void *split_scratch(hipStream_t st, bool allocate)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    const auto key = std::make_pair(dev, st);
    auto it = g_bufs.find(key);
    if (it != g_bufs.end()) return it->second;
    if (!allocate || capturing(st)) return nullptr;
    void *p = nullptr;
    if (hipMalloc(&p, kSplitScratchBytes) != hipSuccess) {
        (void)hipGetLastError();  // leave no error behind for the next call
        return nullptr;
    }
    g_bufs[key] = p;
    return p;
}

void *split_scratch_take(hipStream_t st)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_bufs.find(std::make_pair(dev, st));
    if (it == g_bufs.end()) return nullptr;
    void *p = it->second;
    g_bufs.erase(it);
    return p;
}

}  // namespace gdn
