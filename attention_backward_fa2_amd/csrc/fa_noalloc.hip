// fa_noalloc.hip -- the backward for callers that cannot allocate memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): fa_bwd_noalloc runs exactly the kernels of fa_bwd, with a
// library-owned scratch array in place of the caller's workspace.
//
// The array is a file-scope device variable of FA_BWD_NOALLOC_MAX_WORKSPACE
// bytes; every GPU the library runs on holds its own copy until the process
// ends.  Host code never passes the array's name to a kernel (in host code
// that name is a host-side stand-in, not a device address): its device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and only that address is used.  Calls on one GPU share
// the array, so calls that overlap on one GPU race.  Each call's kernels
// write or clear every part of the workspace they read before reading it
// (the dQ or preprocess step writes the row vectors and the flags, and in
// accumulate mode clears the accumulator and the turn counters), so no call
// depends on what the last one left there.
#include <cstdio>
#include <mutex>

#include "../../include/fa_bwd.h"
#include "fa_internal.h"

namespace fa {
int report_error(int status, const char *msg);   // fa_api.cpp
}

static __device__ __align__(256) unsigned char scratch[FA_BWD_NOALLOC_MAX_WORKSPACE];

namespace {

constexpr size_t kScratchBytes = FA_BWD_NOALLOC_MAX_WORKSPACE;
constexpr int kMaxDevices = 64;

std::mutex g_mu;
void *g_ptr[kMaxDevices];   // device address of `scratch` per device (null until looked up)

fa_status report(fa_status st, const char *msg)
{
    return (fa_status)fa::report_error(st, msg);
}

}  // namespace

extern "C" fa_status fa_bwd_noalloc(const fa_bwd_args *a, void *stream)
{
    if (!a)
        return fa_bwd(a, stream);   // FA_ERR_INVALID_ARG, with its message
    fa_bwd_args b = *a;
    // No dropout keep region: the key-tile kernel draws the keep bits itself
    // (the same bits, bit-identical results).
    b.dropout_keep_max_bytes = 1;
    b.workspace = nullptr;
    b.workspace_bytes = 0;
    // Host-only checks first: nothing touches the GPU before they pass.
    const size_t need = fa_bwd_workspace_size(&b);
    if (need == 0)
        return fa_bwd_validate(&b);   // invalid arguments: status and message say why
    if (need > kScratchBytes) {
        char msg[256];
        snprintf(msg, sizeof msg,
                 "the call needs %zu bytes of workspace, fa_bwd_noalloc has %zu "
                 "(use fa_bwd with a caller-owned workspace)",
                 need, kScratchBytes);
        return report(FA_ERR_WORKSPACE, msg);
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return report(FA_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices)
        return report(FA_ERR_UNSUPPORTED, "device index out of the supported range");
    void *ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        if (!g_ptr[dev]) {
            void *p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return report(FA_ERR_HIP, "hipGetSymbolAddress of the scratch array failed");
            g_ptr[dev] = p;
        }
        ptr = g_ptr[dev];
    }
    b.workspace = ptr;
    b.workspace_bytes = kScratchBytes;
    return fa_bwd(&b, stream);
}
