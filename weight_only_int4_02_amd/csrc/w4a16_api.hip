// C ABI of libw4a16 (declared in include/w4a16.h): host checks, the gfx950
// architecture gate, the choice of kernel, and launches on the caller's stream.
//
// The architecture gate mirrors AutoAWQ issue "Add unit/integration testing":
// a kernel built around one GPU generation's matrix instructions is refused on
// any other, with an explicit error instead of a failed launch.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "w4a16.h"
#include "w4a16_internal.hpp"

using namespace w4a16;

// ---------------------------------------------------------------------------
// Scratch of w4a16_gemm_noalloc: the split-K partial sums live in this
// file-scope device array instead of a caller's workspace.  Each GPU the
// library runs on holds its own copy (W4A16_NOALLOC_SCRATCH_BYTES) until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device array: its device address is looked up once per device with
// hipGetSymbolAddress (scratch_of_current_device) and only that address is
// ever handed to a kernel.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[W4A16_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[256] = "";

void set_hip_error(const char *what, hipError_t e) {
    snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", what,
             hipGetErrorString(e), (int)e);
}

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950, 2 = another architecture
std::atomic<int> g_arch_state[kMaxDevices];

int32_t arch_gate() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        set_hip_error("hipGetDevice", e);
        return W4A16_ERR_HIP;
    }
    int state = (dev >= 0 && dev < kMaxDevices) ? g_arch_state[dev].load() : 0;
    if (state == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) {
            set_hip_error("hipGetDeviceProperties", e);
            return W4A16_ERR_HIP;
        }
        // gcnArchName looks like "gfx950:sramecc+:xnack-"
        const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                        (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
        state = ok ? 1 : 2;
        if (dev >= 0 && dev < kMaxDevices)
            g_arch_state[dev].store(state);
    }
    return state == 1 ? W4A16_OK : W4A16_ERR_ARCH;
}

std::mutex g_scratch_mu;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (looked up on the first
// call on that device, with it current).
int32_t scratch_of_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        set_hip_error("hipGetDevice", e);
        return W4A16_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        snprintf(g_last_error, sizeof(g_last_error), "device %d beyond the %d the library tracks",
                 dev, kMaxDevices);
        return W4A16_ERR_HIP;
    }
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) {
                set_hip_error("hipGetSymbolAddress(scratch)", e);
                return W4A16_ERR_HIP;
            }
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return W4A16_OK;
}

int32_t finish_launch(const char *what, int err) {
    if (err != (int)hipSuccess) {
        set_hip_error(what, (hipError_t)err);
        return W4A16_ERR_HIP;
    }
    return W4A16_OK;
}

}  // namespace

extern "C" {

const char *w4a16_last_hip_error(void) { return g_last_error; }

int32_t w4a16_device_check(void) { return arch_gate(); }

int32_t w4a16_pack(const uint8_t *codes, int64_t rows, int64_t cols, uint32_t *packed,
                   void *stream) {
    int32_t st = w4a16_check_pack_args(codes, rows, cols, packed);
    if (st)
        return st;
    if ((st = arch_gate()))
        return st;
    (void)hipGetLastError();
    return finish_launch("w4a16_pack", launch_pack(codes, rows, cols, packed, stream));
}

int32_t w4a16_repack(const uint32_t *qpacked, const uint16_t *scales,
                     const uint32_t *zeros, int64_t N, int64_t K, int32_t g,
                     uint32_t flags, void *q_dev, void *s_dev, void *z_dev,
                     void *stream) {
    int32_t st = w4a16_check_repack_args(qpacked, scales, zeros, N, K, g, flags, q_dev,
                                         s_dev, z_dev);
    if (st)
        return st;
    if ((st = arch_gate()))
        return st;
    (void)hipGetLastError();
    Geom geo = make_geom(0, N, K, g, flags);
    return finish_launch("w4a16_repack", launch_repack(qpacked, scales, zeros, geo, q_dev,
                                                       s_dev, z_dev, stream));
}

int32_t w4a16_dequant(const uint32_t *qpacked, const uint16_t *scales,
                      const uint32_t *zeros, int64_t N, int64_t K, int32_t g,
                      uint32_t flags, uint16_t *W, void *stream) {
    int32_t st = w4a16_check_dequant_args(qpacked, scales, zeros, N, K, g, flags, W);
    if (st)
        return st;
    if ((st = arch_gate()))
        return st;
    (void)hipGetLastError();
    Geom geo = make_geom(0, N, K, g, flags);
    return finish_launch("w4a16_dequant",
                         launch_dequant(qpacked, scales, zeros, geo, W, stream));
}

int32_t w4a16_quantize(const uint16_t *W, int64_t N, int64_t K, int32_t g, uint32_t flags,
                       uint32_t *qpacked, uint16_t *scales, uint32_t *zeros, void *stream) {
    int32_t st = w4a16_check_quantize_args(W, N, K, g, flags, qpacked, scales, zeros);
    if (st)
        return st;
    if ((st = arch_gate()))
        return st;
    (void)hipGetLastError();
    Geom geo = make_geom(0, N, K, g, flags);
    return finish_launch("w4a16_quantize",
                         launch_quantize(W, geo, qpacked, scales, zeros, stream));
}

int32_t w4a16_gemm(const uint16_t *X, int64_t M, int64_t K, const void *q_dev,
                   const void *s_dev, const void *z_dev, int64_t N, int32_t g,
                   uint32_t flags, uint16_t *Y, void *workspace, size_t workspace_bytes,
                   void *stream) {
    int32_t st = w4a16_check_gemm_args(X, M, K, q_dev, s_dev, z_dev, N, g, flags, Y,
                                       workspace, workspace_bytes);
    if (st)
        return st;
    if ((st = arch_gate()))
        return st;
    (void)hipGetLastError();
    Geom geo = make_geom(M, N, K, g, flags);
    GemmPlan plan = plan_gemm(geo, flags);
    return finish_launch("w4a16_gemm", launch_gemm(X, q_dev, s_dev, z_dev, geo, plan, Y,
                                                   workspace, stream));
}

int32_t w4a16_gemm_noalloc(const uint16_t *X, int64_t M, int64_t K, const void *q_dev,
                           const void *s_dev, const void *z_dev, int64_t N, int32_t g,
                           uint32_t flags, uint16_t *Y, void *stream) {
    // the shape and flag checks, and the scratch this call needs
    size_t need = 0;
    int32_t st = w4a16_gemm_workspace_size(M, N, K, g, flags, &need);
    if (st)
        return st;
    if (need > (size_t)W4A16_NOALLOC_SCRATCH_BYTES) {
        snprintf(g_last_error, sizeof(g_last_error),
                 "w4a16_gemm_noalloc: this call needs %zu bytes of split-K scratch, "
                 "beyond the %zu bytes of the library's static scratch (use w4a16_gemm "
                 "with a workspace)",
                 need, (size_t)W4A16_NOALLOC_SCRATCH_BYTES);
        return W4A16_ERR_WORKSPACE;
    }
    if ((st = arch_gate()))
        return st;
    void *ws = nullptr;
    if (need && (st = scratch_of_current_device(&ws)))
        return st;
    st = w4a16_check_gemm_args(X, M, K, q_dev, s_dev, z_dev, N, g, flags, Y, ws,
                               ws ? (size_t)W4A16_NOALLOC_SCRATCH_BYTES : 0);
    if (st)
        return st;
    (void)hipGetLastError();
    Geom geo = make_geom(M, N, K, g, flags);
    GemmPlan plan = plan_gemm(geo, flags);
    return finish_launch("w4a16_gemm_noalloc",
                         launch_gemm(X, q_dev, s_dev, z_dev, geo, plan, Y, ws, stream));
}

int32_t w4a16_stream_read(const void *a, size_t a_bytes, const void *b, size_t b_bytes,
                          const void *c, size_t c_bytes, uint32_t key, uint32_t *sink,
                          void *stream) {
    if (!sink || (a_bytes && !a) || (b_bytes && !b) || (c_bytes && !c))
        return W4A16_ERR_NULL;
    if ((a_bytes | b_bytes | c_bytes) % 16 != 0 || a_bytes + b_bytes + c_bytes == 0)
        return W4A16_ERR_SHAPE;
    if (((uintptr_t)a | (uintptr_t)b | (uintptr_t)c) & 15u)
        return W4A16_ERR_ALIGN;
    int32_t st = arch_gate();
    if (st)
        return st;
    (void)hipGetLastError();
    return finish_launch("w4a16_stream_read", launch_stream_read(a, a_bytes, b, b_bytes, c, c_bytes,
                                                                 key, sink, stream));
}

}  // extern "C"
