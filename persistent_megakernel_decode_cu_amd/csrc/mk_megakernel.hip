// mk_megakernel.hip - host side of the resident decode interpreter: picks the
// kernel variant (padded batch, q heads per kv head), sets its LDS size,
// checks co-residency and launches it cooperatively. The device code is in
// mk_interp.h, instantiated by mk_interp_b{1,2,4,8}.hip.
#include <algorithm>
#include <mutex>

#include "mk_device.h"

namespace mk {

const void *interp_kernel_b1(int G);
const void *interp_kernel_b2(int G);
const void *interp_kernel_b4(int G);
const void *interp_kernel_b8(int G);

// Scratch for callers that cannot allocate (mk_decode_step_static): the
// exchange words and counters of one step in a file-scope device array, one
// copy per device, alive until the process ends and shared by every such
// call on that device. Host code never passes the array's name to a kernel
// (on the host it is only a stand-in): static_scratch_setup looks its device
// address up once per device and static_scratch returns that address.
static __device__ __align__(256) uint64_t scratch[STATIC_SCRATCH_BYTES / 8];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};

}  // namespace

hipError_t static_scratch_setup(int device) {
    if (device < 0 || device >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[device]) return hipSuccess;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = p;
    return hipSuccess;
}

void *static_scratch(int device) {
    if (device < 0 || device >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_ptr[device];
}

namespace {

const void *kernel_for(int B, int G) {
    if (B <= 1) return interp_kernel_b1(G);
    if (B <= 2) return interp_kernel_b2(G);
    if (B <= 4) return interp_kernel_b4(G);
    return interp_kernel_b8(G);
}

}  // namespace

bool megakernel_supports(int B, int G) { return B >= 1 && B <= MAX_B && kernel_for(B, G) != nullptr; }

hipError_t setup_megakernel(int B, int G, int lds_bytes) {
    const void *k = kernel_for(B, G);
    if (!k) return hipErrorInvalidValue;
    return hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
}

hipError_t megakernel_occupancy(int B, int G, int lds_bytes, int *blocks_per_cu) {
    const void *k = kernel_for(B, G);
    if (!k) return hipErrorInvalidValue;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, k, BLOCK_THREADS, lds_bytes);
}

// Plain fill kernel: clears device words on a stream without hipMemsetAsync,
// whose nodes have given wrong results on graph replays after the first.
__global__ __launch_bounds__(256) void mk_fill_u32(uint32_t *p, size_t n, uint32_t v) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = v;
}

hipError_t fill_u32(uint32_t *p, size_t n, uint32_t v, hipStream_t s) {
    const unsigned blocks = (unsigned)std::min<size_t>(1024, (n + 255) / 256);
    hipLaunchKernelGGL(mk_fill_u32, dim3(blocks ? blocks : 1), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t launch_megakernel(const KParams &p, int lds_bytes, hipStream_t s) {
    const void *k = kernel_for(p.B, p.nq / p.nkv);
    if (!k) return hipErrorInvalidValue;
    KParams arg = p;
    void *args[] = {&arg};
    return hipLaunchCooperativeKernel(k, dim3(p.n_cus), dim3(BLOCK_THREADS), args, (unsigned)lds_bytes, s);
}

}  // namespace mk
