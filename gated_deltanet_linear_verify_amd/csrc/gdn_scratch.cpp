// gdn_scratch.cpp - the readout scratch of the row-split verify: one device buffer per (device,
// stream), so that calls on different streams never share one.  A buffer is allocated on the first
// split launch on its stream, outside stream capture.  Under capture only a buffer reserved for
// capture is used (gdn_graph reserves one for its private capture stream and keeps it for the
// graph's lifetime); a stream's own buffer is not, since a graph recorded with it could be replayed
// on another stream alongside that stream's later calls.  Without one the launcher takes the
// unsplit path, with the same results bit for bit.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <utility>

#include "gdn_internal.h"

namespace gdn {
namespace {

struct Buf {
    void *p;
    bool for_capture;  // reserved for a capture stream (usable under capture)
};
std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Buf> g_bufs;

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
    const bool cap = capturing(st);
    auto it = g_bufs.find(key);
    if (it != g_bufs.end()) return !cap || it->second.for_capture ? it->second.p : nullptr;
    if (!allocate || cap) return nullptr;
    void *p = nullptr;
    if (hipMalloc(&p, kSplitScratchBytes) != hipSuccess) {
        (void)hipGetLastError();  // leave no error behind for the next call
        return nullptr;
    }
    g_bufs[key] = Buf{p, false};
    return p;
}

bool split_scratch_reserve(hipStream_t st)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    std::lock_guard<std::mutex> lock(g_mu);
    const auto key = std::make_pair(dev, st);
    auto it = g_bufs.find(key);
    if (it != g_bufs.end()) {
        it->second.for_capture = true;
        return true;
    }
    if (capturing(st)) return false;
    void *p = nullptr;
    if (hipMalloc(&p, kSplitScratchBytes) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    g_bufs[key] = Buf{p, true};
    return true;
}

void *split_scratch_take(hipStream_t st)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_bufs.find(std::make_pair(dev, st));
    if (it == g_bufs.end()) return nullptr;
    void *p = it->second.p;
    g_bufs.erase(it);
    return p;
}

}  // namespace gdn
