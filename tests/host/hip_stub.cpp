// Test-only stand-ins for the HIP runtime entry points that the library's
// kernel launchers call once their sources are compiled for the host alone
// (hipcc --offload-host-only).  Linked with those objects, the host layer
// (argument checks, schedules, launch slicing) runs on a machine without a
// GPU, under the address and undefined-behaviour sanitizers: every kernel
// launch is recorded here instead of executed.
#include <hip/hip_runtime.h>

#include <map>
#include <string.h>

#include "hip_stub.hpp"

namespace stub {

std::vector<Launch> launches;
int fail_on_call = 0;

namespace {
std::map<const void *, std::string> &names() {
    static std::map<const void *, std::string> m;
    return m;
}
dim3 cfg_grid, cfg_block;
size_t cfg_shm = 0;
hipStream_t cfg_stream = nullptr;

// Index of the int64 first-workgroup argument of each sliced kernel.
int block0_arg(const std::string &name) {
    static const struct {
        const char *kernel;
        int arg;
    } table[] = {{"k_fill", 6},          {"k_step_indep", 6}, {"k_step_chain", 8},
                 {"k_seam_project", 4},  {"k_seam_disc", 5},  {"k_seam_mean_abs", 5},
                 {"k_mds", 6},           {"k_stitch", 6}};
    for (const auto &t : table)
        if (name.find(t.kernel) != std::string::npos) return t.arg;
    return -1;
}
}  // namespace

void reset() {
    launches.clear();
    fail_on_call = 0;
}

}  // namespace stub

extern "C" {

void **__hipRegisterFatBinary(const void *) {
    static void *handle = nullptr;
    return &handle;
}

void __hipUnregisterFatBinary(void **) {}

void __hipRegisterFunction(void **, const void *host_function, char *, const char *device_name, unsigned int, uint3 *,
                           uint3 *, dim3 *, dim3 *, int *) {
    stub::names()[host_function] = device_name;
}

void __hipRegisterVar(void **, void *, char *, char *, int, size_t, int, int) {}

hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t shm, hipStream_t stream) {
    stub::cfg_grid = grid;
    stub::cfg_block = block;
    stub::cfg_shm = shm;
    stub::cfg_stream = stream;
    return hipSuccess;
}

hipError_t __hipPopCallConfiguration(dim3 *grid, dim3 *block, size_t *shm, hipStream_t *stream) {
    *grid = stub::cfg_grid;
    *block = stub::cfg_block;
    *shm = stub::cfg_shm;
    *stream = stub::cfg_stream;
    return hipSuccess;
}

hipError_t hipLaunchKernel(const void *function, dim3 grid, dim3 block, void **args, size_t shm, hipStream_t) {
    stub::Launch l;
    const auto it = stub::names().find(function);
    l.kernel = it == stub::names().end() ? "?" : it->second;
    l.grid = grid.x;
    l.block = block.x;
    l.grid_yz = grid.y * grid.z;
    l.shm = shm;
    const int a = stub::block0_arg(l.kernel);
    if (a >= 0) memcpy(&l.block0, args[a], sizeof l.block0);
    stub::launches.push_back(l);
    return hipSuccess;
}

hipError_t hipGetLastError(void) {
    if (stub::fail_on_call > 0 && --stub::fail_on_call == 0) return hipErrorInvalidConfiguration;
    return hipSuccess;
}

const char *hipGetErrorString(hipError_t) { return "error injected by the host test"; }

}  // extern "C"
