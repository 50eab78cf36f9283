// lce_noalloc.hip -- the forward without a plan and without any device allocation, for callers
// that cannot allocate: code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc.
//
// It runs the two-launch gather-add stage on the streaming engine (user tiles into the fp32
// partial P_u, then the candidates with P_u[map[b]] added in the epilogue; stream order
// publishes P_u).  P_u, and the error word the candidate kernel writes, live in `scratch`, a
// file-scope device array: every GPU the library runs on holds its own copy until the process
// ends, at its own address, found once per device with hipGetSymbolAddress while that device is
// current.  Host code uses that address, never the array's name (which in host code is only a
// host-side stand-in).  Every call on a GPU shares that GPU's array: calls that overlap on one
// GPU (two streams, or two threads) race on P_u.
#include <algorithm>
#include <mutex>

#include "ikbo.h"
#include "fa_internal.h"
#include "lce_internal.h"

namespace ikbo {
namespace {

constexpr size_t kScratchBytes = IKBO_NOALLOC_SCRATCH_BYTES;
constexpr size_t kErrOff = 0;     // the candidate kernel's error word (written, never read back)
constexpr size_t kPuOff = 256;    // P_u [B_u][M][D] fp32
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceScratch {
    unsigned char *ptr = nullptr;   // device address of this device's `scratch`
    int n_cu = 0;
    int max_lds = 0;
};

std::mutex g_scratch_mu;
DeviceScratch g_scratch[kMaxDevices];

// The scratch address and the device limits of `dev` (the current device), looked up on the
// first call on that device.
int device_scratch(int dev, DeviceScratch &out) {
    if (dev < 0 || dev >= kMaxDevices) return status_fail(IKBO_ERR_UNSUPPORTED, "device index out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    DeviceScratch &d = g_scratch[dev];
    if (d.ptr == nullptr) {
        void *ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        int n_cu = 0, max_lds = 0;
        e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(CUs)");
        e = hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(LDS)");
        d.n_cu = n_cu;
        d.max_lds = max_lds;
        d.ptr = static_cast<unsigned char *>(ptr);
    }
    out = d;
    return IKBO_OK;
}

int ceil_div_i(int a, int b) { return (a + b - 1) / b; }

}  // namespace
}  // namespace ikbo

using namespace ikbo;

extern "C" int ikbo_lce_forward_noalloc(const void *U, const void *C, const int32_t *map, const void *W_u,
                                        const void *W_c, void *Y, int B_u, int B_c, int K_u, int K_c, int M,
                                        int D, void *stream) {
    if (B_c < 0 || B_u < 1 || K_u < 1 || K_c < 1 || M < 1 || D < 1) return IKBO_ERR_INVALID_ARG;
    if (B_c == 0) return IKBO_OK;
    if (!U || !C || !map || !W_u || !W_c || !Y) return IKBO_ERR_INVALID_ARG;
    if (((reinterpret_cast<uintptr_t>(U) | reinterpret_cast<uintptr_t>(C) | reinterpret_cast<uintptr_t>(Y) |
          reinterpret_cast<uintptr_t>(W_u) | reinterpret_cast<uintptr_t>(W_c)) & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(map) & 3u) != 0)
        return IKBO_ERR_ALIGNMENT;
    if (!stream_supported(D))
        return status_fail(IKBO_ERR_UNSUPPORTED, "ikbo_lce_forward_noalloc: D must be 32, 64, 128, 160 or 192");
    // Byte offsets within one fp32 [M][D] matrix and one [K][D] matrix are 32-bit.
    if ((long long)M * D * 4 >= (1LL << 31) || (long long)(K_u > K_c ? K_u : K_c) * D * 2 >= (1LL << 31))
        return status_fail(IKBO_ERR_UNSUPPORTED, "ikbo_lce_forward_noalloc: a matrix exceeds 2 GiB");
    if ((long long)B_u * M * D * 4 > (long long)(kScratchBytes - kPuOff))
        return status_fail(IKBO_ERR_UNSUPPORTED,
                           "ikbo_lce_forward_noalloc: B_u*M*D*4 bytes of user partial exceed the scratch array");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    DeviceScratch ds;
    int st = device_scratch(dev, ds);
    if (st != IKBO_OK) return st;

    const int n_rb = ceil_div_i(M, 16), n_cb = D / 16;
    const int mb = stream_choose_mb(n_rb, stream_max_mb(D), B_c, ds.n_cu * (kStreamBlock / 64));
    const int n_mc = ceil_div_i(n_rb, mb);
    StreamArgs a{};
    a.U = static_cast<const uint16_t *>(U);
    a.C = static_cast<const uint16_t *>(C);
    a.W_u = static_cast<const uint16_t *>(W_u);
    a.W_c = static_cast<const uint16_t *>(W_c);
    a.map = map;
    a.out = Y;
    a.P_u = reinterpret_cast<float *>(ds.ptr + kPuOff);
    a.flags = nullptr;
    a.err = reinterpret_cast<uint32_t *>(ds.ptr + kErrOff);
    a.B_u = B_u; a.M = M; a.D = D;
    a.K_u = K_u; a.K_c = K_c; a.K_wc = K_c;
    a.n_ks_u = ceil_div_i(K_u, 32); a.n_ks_c = ceil_div_i(K_c, 32);
    a.n_rb = n_rb; a.n_cb = n_cb; a.n_mc = n_mc;
    a.xcd_order = 1;
    a.wait_flags = 0;
    a.tile_waves = 4;
    a.spin_limit = 0;
    a.debug_flags = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto launch = [&](StreamArgs x, const char *what) -> int {
        stream_lds_layout(x);
        const size_t lds = stream_lds_bytes(x);
        if (lds > (size_t)ds.max_lds)
            return status_fail(IKBO_ERR_UNSUPPORTED, "ikbo_lce_forward_noalloc: the LDS does not hold the staged operands");
        const int bpc = stream_blocks_per_cu(EPI_ADD_USER, D, mb, lds);
        if (bpc < 1) return status_fail(IKBO_ERR_UNSUPPORTED, "ikbo_lce_forward_noalloc: kernel does not fit a CU");
        const int blocks = std::max(ceil_div_i(x.n_units, kStreamBlock / 64), ceil_div_i(x.n_utiles, x.tile_waves));
        const int grid = std::max(1, std::min(ds.n_cu * bpc, blocks));
        const hipError_t le = launch_stream(EPI_ADD_USER, mb, x, grid, s);
        return le == hipSuccess ? IKBO_OK : hip_fail(le, what);
    };
    StreamArgs u = a;
    u.n_utiles = B_u * n_rb * n_cb;
    u.n_units = 0;
    if ((st = launch(u, "user tiles")) != IKBO_OK) return st;
    StreamArgs c = a;
    c.n_utiles = 0;
    c.n_units = B_c * n_mc;
    return launch(c, "candidates");
}
