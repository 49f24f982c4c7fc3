// Test-only record of the kernel launches the library's host layer makes when
// its sources are compiled for the host alone and linked with hip_stub.cpp.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

namespace stub {

struct Launch {
    std::string kernel;   // device name as registered (mangled)
    uint32_t grid = 0;    // workgroups in the dispatch (x)
    uint32_t block = 0;   // lanes per workgroup (x)
    uint32_t grid_yz = 0; // grid.y * grid.z (must stay 1)
    int64_t block0 = -1;  // the slice's first logical workgroup (-1: the kernel takes none)
    size_t shm = 0;
};

extern std::vector<Launch> launches;
// hipGetLastError returns an error on its n-th call from now (1 = the next);
// 0 never.
extern int fail_on_call;

void reset();

}  // namespace stub
