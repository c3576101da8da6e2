// HSA runtime helpers for copies that bypass HIP's queues
// (hsa_amd_memory_async_copy on the DMA engines, completion signals).
#pragma once

#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

namespace moe {

// The HSA agents of HIP device `device` (matched by PCI domain, bus and
// device) and of the host (the first CPU agent), for
// hsa_amd_memory_async_copy.  The caller has called hsa_init.  False if
// either is not found.
bool hsa_agents_of(int device, hsa_agent_t* gpu, hsa_agent_t* cpu);

}  // namespace moe
