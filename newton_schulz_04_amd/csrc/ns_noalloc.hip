// ns_noalloc.hip -- ns_orthogonalize_batched_noalloc: the batched call for
// callers that cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The workspace and the metadata block live in `scratch`, a file-scope device
// array of NS_NOALLOC_SCRATCH_BYTES that each device holds from the moment
// this code object is loaded on it until the process ends. Its device address
// comes from hipGetSymbolAddress, once per device, on the first call on that
// device; host code uses only that address, never the array's name. The
// metadata (descriptors and tile lists) goes up through kernel arguments
// (k_put, 2 KB per launch), so no pinned staging buffer is
// needed and the host image can be reused as soon as the launch returns.
//
// Nothing in the workspace has to start at zero: the normalize pass writes
// all of X including its zero padding, and the products write every element
// of A and B before they are read (as with the allocated workspace of
// ns_orthogonalize_batched).
#include <hip/hip_runtime.h>

#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "ns.h"
#include "ns_enqueue.h"
#include "ns_plan.h"

// The scratch array. In host code its name is a host-side stand-in, not a
// device address: only the address hipGetSymbolAddress returns is passed on.
static __device__ __align__(256) char scratch[NS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = NS_NOALLOC_SCRATCH_BYTES;
constexpr size_t kPieceBytes = 2048;          // metadata bytes per k_put launch
constexpr int kPieceVec = kPieceBytes / 16;   // 16-byte words per piece

struct alignas(16) MetaPiece {
    uint4 w[kPieceVec];
};

// dst[0 .. nvec) = piece.w[0 .. nvec): one workgroup, one 16-byte store per
// thread. dst is 16-byte aligned.
__global__ __launch_bounds__(kPieceVec) void k_put(uint4* __restrict__ dst, const MetaPiece piece, int nvec)
{
    const int t = threadIdx.x;
    if (t < nvec)
        dst[t] = piece.w[t];
}

std::mutex g_mu;
std::map<int, char*> g_base;   // device -> address of its `scratch`

// Device address of this device's scratch array (looked up once per device).
ns_status scratch_base(int dev, char** out)
{
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_base.find(dev);
    if (it != g_base.end()) {
        *out = it->second;
        return NS_OK;
    }
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
        (void)hipGetLastError();
        return ns::hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    }
    g_base[dev] = static_cast<char*>(ptr);
    *out = static_cast<char*>(ptr);
    return NS_OK;
}

}  // namespace

extern "C" ns_status ns_orthogonalize_batched_noalloc(void* const* ptrs, const int64_t* shapes,
                                                      int32_t count, int32_t steps, const float* coeffs,
                                                      int32_t dtype, void* stream)
{
    ns::clear_error();
    ns_status st = ns::validate_batched(ptrs, shapes, count, steps, coeffs, 0, dtype);
    if (st != NS_OK)
        return st;
    bool any = false;
    for (int32_t i = 0; i < count; ++i)
        any = any || (shapes[2 * i] > 0 && shapes[2 * i + 1] > 0);
    if (!any)
        return NS_OK;
    ns::Plan plan;
    std::string err;
    const int rc = ns::make_plan(shapes, count, dtype, &plan, &err);
    if (rc != 0)
        return ns::fail((ns_status)rc, err);
    const size_t meta_off = (plan.data_bytes + 255) / 256 * 256;
    const size_t need = meta_off + plan.meta_end;
    if (need > kScratchBytes)
        return ns::fail(NS_EINVAL, "the batch needs " + std::to_string(need) +
                                       " bytes of workspace; the no-allocation entry point has " +
                                       std::to_string(kScratchBytes));
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return ns::hip_fail(e, "hipGetDevice");
    char* base = nullptr;
    if ((st = scratch_base(dev, &base)) != NS_OK)
        return st;
    char* meta = base + meta_off;
    ns::Layout L;
    L.ptrs = ptrs;
    std::vector<char> img;
    ns::build_meta(plan, L, count, base, meta, &img);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    for (size_t off = 0; off < img.size(); off += kPieceBytes) {
        MetaPiece piece{};
        const size_t n = img.size() - off < kPieceBytes ? img.size() - off : kPieceBytes;
        std::memcpy(&piece, img.data() + off, n);
        hipLaunchKernelGGL(k_put, dim3(1), dim3(kPieceVec), 0, s, reinterpret_cast<uint4*>(meta + off), piece,
                           (int)((n + 15) / 16));
        if ((e = hipGetLastError()) != hipSuccess)
            return ns::hip_fail(e, "metadata upload");
    }
    return ns::enqueue(plan, meta, steps, coeffs, 0, dtype, s);
}
