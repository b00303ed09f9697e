#include "kda_common.hpp"
#include "kda_launch.hpp"
namespace kda {
hipError_t launch_chunk_staged(const ChunkLaunch&) { return hipErrorNotSupported; }
}
