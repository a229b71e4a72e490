// Replay of a recorded decode step with double-buffered host-built tables ("Paged KV Cache
// and Packed Sequence", 5.3: the host builds the small, changing structures and they are
// copied in before the step; with two buffers the host fills the next one while this step
// runs).
//
// The runner holds two graphs (graph j recorded over device buffer j) and two events; the
// caller owns the buffers.  Graph j begins with a copy kernel that reads pinned host buffer
// j through its device view (16-byte loads over the host link) into device buffer j, then
// runs the recorded step.  Per step t (j = t % 2):
//   host:   pkv_runner_host_buffer waits until the replay that last read host buffer j
//           (step t - 2) has run, then the caller fills it;
//   stream: replay graph j, record "consumed j".
// So a step is one graph launch on one stream: no copy engine, no second stream and no
// event between streams (measured on MI355X: the copy-stream upload and the cross-stream
// wait cost more than the copy kernel itself).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>

#include "../../include/pagedkv.h"
#include "pkv_internal.h"

struct pkv_step_runner {
    void* dev[2];
    const void* host[2];
    const void* host_view[2];   // device views of the pinned host buffers
    size_t bytes;
    hipEvent_t consumed[2] = {nullptr, nullptr};
    bool use_rec[2] = {false, false};
    hipGraphExec_t graph[2] = {nullptr, nullptr};
    int capturing = -1;
    int64_t t = 0;
};

namespace {

int rn_fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    pkv::set_error_v(code, fmt, ap);
    va_end(ap);
    return code;
}

int rn_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return PKV_OK;
    return rn_fail(PKV_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

void release(pkv_step_runner* r) {
    for (int j = 0; j < 2; ++j) {
        if (r->use_rec[j]) (void)hipEventSynchronize(r->consumed[j]);
        if (r->graph[j]) (void)hipGraphExecDestroy(r->graph[j]);
        if (r->consumed[j]) (void)hipEventDestroy(r->consumed[j]);
    }
    delete r;
}

}  // namespace

extern "C" {

pkv_step_runner* pkv_runner_create(void* dev0, void* dev1, const void* host0, const void* host1,
                                   size_t bytes) {
    if (!dev0 || !dev1 || !host0 || !host1 || bytes == 0) {
        rn_fail(PKV_ERR_NULL, "runner_create: buffers must be non-NULL and bytes > 0");
        return nullptr;
    }
    if (dev0 == dev1 || host0 == host1) {
        rn_fail(PKV_ERR_SHAPE, "runner_create: the two buffers of each side must differ");
        return nullptr;
    }
    if (bytes % 4) {
        rn_fail(PKV_ERR_SHAPE, "runner_create: bytes must be a multiple of 4 (int32 tables)");
        return nullptr;
    }
    auto* r = new pkv_step_runner();
    r->dev[0] = dev0;
    r->dev[1] = dev1;
    r->host[0] = host0;
    r->host[1] = host1;
    r->bytes = bytes;
    int rc = PKV_OK;
    for (int j = 0; j < 2 && rc == PKV_OK; ++j) {
        void* view = nullptr;
        rc = rn_hip(hipHostGetDevicePointer(&view, const_cast<void*>(r->host[j]), 0),
                    "runner_create: host buffers must be pinned (hipHostMalloc); device view");
        r->host_view[j] = view;
        if (rc == PKV_OK && ((reinterpret_cast<uintptr_t>(view) | reinterpret_cast<uintptr_t>(r->dev[j])) % 16))
            rc = rn_fail(PKV_ERR_ALIGN, "runner_create: buffers must be 16-byte aligned");
        if (rc == PKV_OK)
            rc = rn_hip(hipEventCreateWithFlags(&r->consumed[j], hipEventDisableTiming), "runner_create: event");
    }
    if (rc != PKV_OK) {
        release(r);
        return nullptr;
    }
    return r;
}

int pkv_runner_destroy(pkv_step_runner* r) {
    if (r) release(r);
    return PKV_OK;
}

int pkv_runner_capture_begin(pkv_step_runner* r, int32_t j, void* stream) {
    if (!r || !stream) return rn_fail(PKV_ERR_NULL, "runner_capture_begin: NULL runner or stream");
    if (j < 0 || j > 1) return rn_fail(PKV_ERR_SHAPE, "runner_capture_begin: buffer index %d is not 0 or 1", j);
    if (r->capturing >= 0) return rn_fail(PKV_ERR_SHAPE, "runner_capture_begin: a capture is open");
    if (r->graph[j]) return rn_fail(PKV_ERR_SHAPE, "runner_capture_begin: graph %d already recorded", j);
    int rc = rn_hip(hipStreamBeginCapture((hipStream_t)stream, hipStreamCaptureModeThreadLocal),
                    "runner_capture_begin");
    if (rc != PKV_OK) return rc;
    r->capturing = j;
    // the graph's first node: host buffer j -> device buffer j
    return rn_hip(pkv::launch_host_copy(r->dev[j], r->host_view[j], (int64_t)r->bytes, (hipStream_t)stream),
                  "runner_capture_begin: table copy");
}

int pkv_runner_capture_end(pkv_step_runner* r, void* stream) {
    if (!r || !stream) return rn_fail(PKV_ERR_NULL, "runner_capture_end: NULL runner or stream");
    if (r->capturing < 0) return rn_fail(PKV_ERR_SHAPE, "runner_capture_end: no capture is open");
    const int j = r->capturing;
    r->capturing = -1;
    hipGraph_t g = nullptr;
    int rc = rn_hip(hipStreamEndCapture((hipStream_t)stream, &g), "runner_capture_end: end capture");
    if (rc != PKV_OK) return rc;
    rc = rn_hip(hipGraphInstantiate(&r->graph[j], g, nullptr, nullptr, 0), "runner_capture_end: instantiate");
    (void)hipGraphDestroy(g);
    return rc;
}

void* pkv_runner_graph(pkv_step_runner* r, int32_t j) {
    return (r && j >= 0 && j <= 1) ? (void*)r->graph[j] : nullptr;
}

void* pkv_runner_host_buffer(pkv_step_runner* r) {
    if (!r) {
        rn_fail(PKV_ERR_NULL, "runner_host_buffer: NULL runner");
        return nullptr;
    }
    const int j = (int)(r->t & 1);
    if (r->use_rec[j] && rn_hip(hipEventSynchronize(r->consumed[j]), "runner_host_buffer") != PKV_OK)
        return nullptr;
    return const_cast<void*>(r->host[j]);
}

int pkv_runner_launch(pkv_step_runner* r, void* stream) {
    if (!r) return rn_fail(PKV_ERR_NULL, "runner_launch: NULL runner");
    const int j = (int)(r->t & 1);
    if (!r->graph[j]) return rn_fail(PKV_ERR_SHAPE, "runner_launch: graph %d was not recorded", j);
    hipStream_t s = (hipStream_t)stream;
    int rc = rn_hip(hipGraphLaunch(r->graph[j], s), "runner_launch: replay");
    if (rc == PKV_OK) rc = rn_hip(hipEventRecord(r->consumed[j], s), "runner_launch: record");
    if (rc != PKV_OK) return rc;
    r->use_rec[j] = true;
    ++r->t;
    return PKV_OK;
}

int pkv_upload_kernel(void* dst, const void* src_host, size_t bytes, void* stream) {
    if (bytes == 0) return PKV_OK;
    if (!dst || !src_host) return rn_fail(PKV_ERR_NULL, "upload_kernel: NULL pointer argument");
    if (bytes % 4) return rn_fail(PKV_ERR_SHAPE, "upload_kernel: bytes must be a multiple of 4");
    void* view = nullptr;
    int rc = rn_hip(hipHostGetDevicePointer(&view, const_cast<void*>(src_host), 0),
                    "upload_kernel: src_host must be pinned (hipHostMalloc); device view");
    if (rc != PKV_OK) return rc;
    if ((reinterpret_cast<uintptr_t>(view) | reinterpret_cast<uintptr_t>(dst)) % 16)
        return rn_fail(PKV_ERR_ALIGN, "upload_kernel: buffers must be 16-byte aligned");
    return rn_hip(pkv::launch_host_copy(dst, view, (int64_t)bytes, (hipStream_t)stream), "upload_kernel");
}

}  // extern "C"
