// qsa_internal.h -- what every HIP source of libqsa.so includes: the public
// ABI types, the launcher interface (qsa_launch.h) and the device helpers.
// Not part of the public ABI.
#pragma once

#include "qsa.h"
#include "qsa_launch.h"
#include "qsa_device.h"
